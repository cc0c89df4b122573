// Tree preparation: validates each sequence's packed tree and inputs and
// derives what the attention and sampling kernels need from the parent array.
//
// The packed tree and its mask follow "LLM speculative decoding: EAGLE"
// (jingming.pro) sec. 4.2 "Attention Mask" and the EAGLE-2 excerpts
// (modelers.csdn.net) sec. 2.3.2: the drafted nodes are flattened into one
// sequence and node j may see the prefix, its ancestors and itself. Here the
// ancestor-or-self set of node j is a 64-bit mask (bit a = node a), and the
// children of every slot are listed in ascending node index, the order in
// which multi-round speculative sampling tests them.
#include "sv_internal.h"

namespace sv {

// One wave per sequence. Writes, for sequence b:
//   anc[b*R + s]        ancestor-or-self mask of slot s (slot 0: 0)
//   nkids[b*R + s]      number of children of slot s
//   kids[(b*R+s)*maxc + i]  i-th child (ascending node index)
//   flags[b]            SV_SEQ_ERR_* bits
//   bar[b]              0 (the sampling walk's barrier counter)
// With `distinct` (siblings drawn without replacement), two children of one
// slot with the same token are an input error for sequences with T > 0.
__global__ __launch_bounds__(64) void k_tree_prep(
    int N, int V, int maxc, int max_prefix, int distinct, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ token, const float* __restrict__ temperature,
    const int32_t* __restrict__ kv_offset, uint64_t* __restrict__ anc,
    int32_t* __restrict__ nkids, int32_t* __restrict__ kids, int32_t* __restrict__ flags,
    int32_t* __restrict__ bar) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int R = N + 1;
  __shared__ int par[kMaxNodes];
  __shared__ int tok[kMaxNodes];
  __shared__ int s_err;
  if (lane == 0) s_err = 0;
  int err = 0;
  if (lane < N) {
    const int p = parent[(size_t)b * N + lane];
    par[lane] = p;
    if (p < -1 || p >= lane) err |= SV_SEQ_ERR_TREE;
    if (token != nullptr) {
      const int t = token[(size_t)b * N + lane];
      tok[lane] = t;
      if (t < 0 || t >= V) err |= SV_SEQ_ERR_TOKEN;
    }
  }
  if (lane == 0) {
    if (temperature != nullptr) {
      const float T = temperature[b];
      if (!(T >= 0.0f) || T == INFINITY) err |= SV_SEQ_ERR_TEMPERATURE;
    }
    if (kv_offset != nullptr) {
      const long long L = (long long)kv_offset[b + 1] - kv_offset[b] - N;
      if (L < 1 || L > max_prefix) err |= SV_SEQ_ERR_PREFIX;
    }
  }
  __syncthreads();
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  const bool tree_ok = (s_err & SV_SEQ_ERR_TREE) == 0;
  if (distinct && token != nullptr && temperature != nullptr && temperature[b] > 0.0f &&
      lane < N && tree_ok) {
    bool dup = false;
    for (int i = 0; i < lane; ++i) dup |= (par[i] == par[lane] && tok[i] == tok[lane]);
    if (dup) atomicOr(&s_err, SV_SEQ_ERR_TOKEN);
  }

  // children lists, one slot per lane (R may exceed 64 by one)
  for (int s = lane; s < R; s += 64) {
    int cnt = 0;
    if (tree_ok) {
      for (int j = s; j < N; ++j) {          // a child of slot s has index >= s
        if (par[j] + 1 == s) {
          if (cnt < maxc) kids[((size_t)b * R + s) * maxc + cnt] = j;
          ++cnt;
        }
      }
    }
    if (cnt > maxc) atomicOr(&s_err, SV_SEQ_ERR_TREE);
    nkids[(size_t)b * R + s] = cnt < maxc ? cnt : maxc;
  }

  // ancestor-or-self masks; parent[j] < j bounds the walk by j steps
  if (lane < N) {
    uint64_t m = 0;
    if (tree_ok) {
      int x = lane;
      while (x >= 0) {
        m |= (uint64_t)1 << x;
        x = par[x];
      }
    }
    anc[(size_t)b * R + lane + 1] = m;
  }
  if (lane == 0) anc[(size_t)b * R] = 0;
  __syncthreads();
  if (lane == 0) {
    flags[b] = s_err;
    bar[b] = 0;
  }
}

hipError_t launch_tree_prep(const Plan& P, const Args& a, bool check_prefix, hipStream_t s) {
  hipLaunchKernelGGL(k_tree_prep, dim3(P.B), dim3(64), 0, s, P.N, P.V, P.max_children,
                     P.max_prefix, P.sampling == SV_SAMPLE_DISTINCT ? 1 : 0, a.parent, a.token,
                     a.temperature,
                     check_prefix ? a.kv_offset : nullptr, ws_anc(P, a.ws), ws_nkids(P, a.ws),
                     ws_kids(P, a.ws), ws_flags(P, a.ws), ws_bar(P, a.ws));
  return hipGetLastError();
}

}  // namespace sv
