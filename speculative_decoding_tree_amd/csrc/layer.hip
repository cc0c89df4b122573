// The full verify-layer share: projections, rotary positions by tree depth,
// tree attention, output projection and the residual that feeds the LM head.
//
// What is computed ("LLM speculative decoding: EAGLE", jingming.pro, sec. 3.1
// and 4.2; "EAGLE (ICML 2024) close reading", edgeai1.github.io, sec. 5: the
// tree's position ids must be set correctly): for every slot of a sequence,
// q = h Wq^T, and for every node k = h Wk^T, v = h Wv^T; q and k are rotated
// by their position (root L - 1, node j at L - 1 + depth(j), so each
// root-to-node path sees the positions of an ordinary decode); the nodes'
// rotated K and V go to their cache rows L + j; tree attention over the
// prefix and the ancestors; h' = h + attn Wo^T is the LM head's input. The
// root's K/V is the cache's row L - 1 (written by the previous step).
//
// Rotary layout: dimension pairs (i, i + D/2), i < D/2, rotated by
// pos * theta^(-2i/D). The angle is formed and reduced modulo 2 pi in fp64
// (positions reach tens of thousands), then sin/cos in fp32.
//
// Kernels (the projections use the library's bf16 GEMM, fp32 out: Q, K and V
// as one launch over three column segments, O with its K split in two so
// both launches fill the chip):
//   k_rope_scatter  one block per slot row: q -> bf16 query buffer; for node
//                   slots K and V -> bf16 cache rows.
//   (tree attention writes its output as bf16, the O GEMM's input, and as
//   fp32 only into the caller's attn_out)
//   k_residual      h' = bf16(h + (o_0 + o_1)), the two K halves of o added
//                   in a fixed order.
#include "sv_internal.h"

namespace sv {

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

struct LayerParams {
  const float* q32;        // [M, Hq*D]
  const float* k32;        // [M, Hkv*D]
  const float* v32;        // [M, Hkv*D]
  uint16_t* q16;           // [M, Hq*D] bf16
  uint16_t* kv;            // cache [rows, 2, Hkv, D] bf16
  const int32_t* kv_offset;
  const uint64_t* anc;     // [M] ancestor masks (slot 0: 0)
  const int32_t* flags;
  int N, R, Hq, Hkv, D;
  double log2_theta;
};

// one block of D/2 threads per slot row; thread i owns dimension pair (i, i + D/2)
__global__ void k_rope_scatter(LayerParams p) {
  const int row = blockIdx.x;
  const int b = row / p.R, s = row % p.R;
  const int i = threadIdx.x;
  const int half = p.D / 2;
  if (p.flags[b] & kSeqErrMask) return;
  const int L = p.kv_offset[b + 1] - p.kv_offset[b] - p.N;
  const int depth = (s == 0) ? 0 : __popcll(p.anc[row]);
  const double pos = (double)(L - 1 + depth);
  const double inv = exp2(-2.0 * (double)i / (double)p.D * p.log2_theta);
  const double two_pi = 6.283185307179586476925286766559;
  double ang = pos * inv;
  ang -= two_pi * floor(ang / two_pi);
  float sn, cs;
  __sincosf((float)ang, &sn, &cs);
  for (int h = 0; h < p.Hq; ++h) {
    const float* src = p.q32 + (size_t)row * p.Hq * p.D + h * p.D;
    const float a = src[i], c = src[i + half];
    uint16_t* dst = p.q16 + (size_t)row * p.Hq * p.D + h * p.D;
    dst[i] = to_bf16_bits(a * cs - c * sn);
    dst[i + half] = to_bf16_bits(a * sn + c * cs);
  }
  if (s == 0) return;
  const size_t crow = (size_t)p.kv_offset[b] + L + (s - 1);
  for (int g = 0; g < p.Hkv; ++g) {
    const float* ks = p.k32 + (size_t)row * p.Hkv * p.D + g * p.D;
    const float* vs = p.v32 + (size_t)row * p.Hkv * p.D + g * p.D;
    uint16_t* kd = p.kv + ((crow * 2 + 0) * p.Hkv + g) * p.D;
    uint16_t* vd = p.kv + ((crow * 2 + 1) * p.Hkv + g) * p.D;
    const float a = ks[i], c = ks[i + half];
    kd[i] = to_bf16_bits(a * cs - c * sn);
    kd[i + half] = to_bf16_bits(a * sn + c * cs);
    vd[i] = to_bf16_bits(vs[i]);
    vd[i + half] = to_bf16_bits(vs[i + half]);
  }
}

__global__ void k_residual(const uint16_t* __restrict__ h, const float* __restrict__ o,
                           const float* __restrict__ o2, uint16_t* __restrict__ out, size_t n) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const float ov = (o2 != nullptr) ? o[e] + o2[e] : o[e];
    out[e] = to_bf16_bits(bf16_bits_to_f32(h[e]) + ov);
  }
}

// Workspace of the layer share: tree prep and attention (the verification
// plan's first region), the tree prep's per-sequence counters right after
// it, then the projections' buffers.
static size_t layer_base(const Plan& P) {
  return (P.bytes_attn_end + sizeof(int32_t) * P.B + 255) & ~(size_t)255;
}

size_t layer_workspace_bytes(const Plan& P) {
  const size_t M = (size_t)P.B * P.R;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return layer_base(P) + up(M * P.Hq * P.D * 4) + 2 * up(M * P.Hkv * P.D * 4) +
         up(M * P.Hq * P.D * 2) + up(M * P.Hq * P.D * 2) + 2 * up(M * P.d * 4);
}

hipError_t launch_layer_share(const Plan& P0, const Args& a, const void* wq, const void* wk,
                              const void* wv, const void* wo, double theta, void* kv,
                              void* out_hidden, float* attn_out, hipStream_t s) {
  Plan P = P0;
  P.off_bar = P.bytes_attn_end;     // inside the layer's workspace
  const size_t M = (size_t)P.B * P.R;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* w = a.ws + layer_base(P);
  float* q32 = (float*)w;            w += up(M * P.Hq * P.D * 4);
  float* k32 = (float*)w;            w += up(M * P.Hkv * P.D * 4);
  float* v32 = (float*)w;            w += up(M * P.Hkv * P.D * 4);
  uint16_t* q16 = (uint16_t*)w;      w += up(M * P.Hq * P.D * 2);
  uint16_t* att16 = (uint16_t*)w;    w += up(M * P.Hq * P.D * 2);
  float* o32 = (float*)w;           // two K halves, M * d apart
  if (launch_tree_prep(P, a, true, s, false) != hipSuccess) return hipErrorLaunchFailure;
  GemmSegs qkv{};
  qkv.count = 3;
  qkv.w[0] = (const bf16_t*)wq;
  qkv.w[1] = (const bf16_t*)wk;
  qkv.w[2] = (const bf16_t*)wv;
  qkv.c[0] = q32;
  qkv.c[1] = k32;
  qkv.c[2] = v32;
  qkv.n[0] = P.Hq * P.D;
  qkv.n[1] = qkv.n[2] = P.Hkv * P.D;
  if (launch_gemm_segments((int)M, P.d, a.hidden, qkv, 1, s) != hipSuccess)
    return hipErrorLaunchFailure;
  LayerParams lp{q32, k32, v32, q16, (uint16_t*)kv, a.kv_offset, ws_anc(P, a.ws),
                 ws_flags(P, a.ws), P.N, P.R, P.Hq, P.Hkv, P.D, log2(theta)};
  hipLaunchKernelGGL(k_rope_scatter, dim3((unsigned)M), dim3(P.D / 2), 0, s, lp);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  // attention writes the O projection's bf16 input itself, and fp32 only
  // when the caller asked for attn_out
  Args at = a;
  at.kv = kv;
  at.hidden = q16;
  at.attn_out = attn_out;
  at.attn_out16 = att16;
  if (launch_attention(P, at, s) != hipSuccess) return hipErrorLaunchFailure;
  const size_t nd = M * P.d;
  GemmSegs op{};
  op.count = 1;
  op.w[0] = (const bf16_t*)wo;
  op.c[0] = o32;
  op.n[0] = P.d;
  op.split_stride[0] = nd;
  const int ksplit = (M >= 512 && (P.Hq * P.D) % 128 == 0) ? 2 : 1;
  if (launch_gemm_segments((int)M, P.Hq * P.D, att16, op, ksplit, s) != hipSuccess)
    return hipErrorLaunchFailure;
  hipLaunchKernelGGL(k_residual, dim3(2048), dim3(256), 0, s, (const uint16_t*)a.hidden, o32,
                     ksplit == 2 ? o32 + nd : (const float*)nullptr, (uint16_t*)out_hidden, nd);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return hipMemcpyAsync(a.seq_status, ws_flags(P, a.ws), sizeof(int32_t) * P.B,
                        hipMemcpyDeviceToDevice, s);
}

}  // namespace sv
