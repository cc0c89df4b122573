// Device helpers shared by the kernels whose workgroups split one sequence's
// vocabulary passes and meet at a sequence-wide barrier (the sampling walk
// and its top-k / top-p selection).
#pragma once

#include "sv_internal.h"

namespace sv {

constexpr int kThreads = 256;                              // threads per walk workgroup
constexpr int kSpinLimit = 1 << 22;                        // bounded barrier wait

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Four values of one 256-token tile for this lane (tokens in ascending order
// within the lane); out-of-range tokens read as -inf.
template <bool VEC>
__device__ __forceinline__ void load_tile4(const float* z, int v0, int V, float (&x)[4],
                                           int (&idx)[4]) {
  const int lane = lane_id();
  if (VEC) {
    const int v = v0 + 4 * lane;
    if (v + 3 < V) {
      const float4 f = *(const float4*)(z + v);
      x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (v + e < V) ? z[v + e] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) idx[e] = v + e;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v0 + lane + 64 * e;
      idx[e] = v;
      x[e] = (v < V) ? z[v] : -INFINITY;
    }
  }
}

// Data exchanged between the workgroups of a sequence (partials, tile masses)
// goes through agent-scope atomic stores and loads, which read and write at
// the device's coherence point; ordinary loads of the read-only logits keep
// their caches. No cache-wide fence is needed.
__device__ __forceinline__ void xstore(float* ptr, float v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float xload(const float* ptr) {
  return __hip_atomic_load(const_cast<float*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename U>
__device__ __forceinline__ void xstore_u(U* ptr, U v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename U>
__device__ __forceinline__ U xload_u(const U* ptr) {
  return __hip_atomic_load(const_cast<U*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All-to-all exchange of NW floats per workgroup of a sequence, without a
// counter: workgroup blockIdx.x stores each value as a 64-bit word (phase,
// value) in its slot of `buf` (kXWords words per slot), and wave 0 of every
// workgroup polls the G slots (lane w: workgroup w) until every word carries
// `phase`, which delivers the values with the wait; it leaves them in
// vals[w][k] (LDS) for every wave. Every wave's earlier stores (a pass's tile
// masses) complete before the words are stored, so a workgroup that has seen
// a phase also sees them. Phases grow by one per exchange and start at 1 (the
// slots are zeroed before the walk), and callers alternate between two
// buffers by phase parity: a workgroup cannot publish phase k + 2 before every
// workgroup has published k + 1, which each does only after reading phase k.
// False when the bounded wait gave up.
constexpr int kXWords = kWalkXWords;
template <int NW>
__device__ inline bool tagged_exchange(unsigned long long* buf, unsigned phase,
                                       const float (&mine)[NW], int G, float (*vals)[kXWords],
                                       int* s_flag) {
  static_assert(NW >= 1 && NW <= kXWords, "words per slot");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < NW; ++k)
      xstore_u(buf + (size_t)blockIdx.x * kXWords + k,
               ((unsigned long long)phase << 32) | __float_as_uint(mine[k]));
  }
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    bool ok = true;
    if (lane < G) {
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        int spins = 0;
        unsigned long long w = xload_u(buf + (size_t)lane * kXWords + k);
        while ((unsigned)(w >> 32) != phase) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            ok = false;
            break;
          }
          w = xload_u(buf + (size_t)lane * kXWords + k);
        }
        vals[lane][k] = __uint_as_float((unsigned)w);
      }
    }
    const bool all = __ballot(!ok) == 0ull;
    if (lane == 0) *s_flag = all ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Tiles [t0, t1) of the vocabulary handled by workgroup wg of G.
__device__ __forceinline__ void wg_tiles(int CT, int G, int wg, int* t0, int* t1) {
  const int per = (CT + G - 1) / G;
  *t0 = min(CT, wg * per);
  *t1 = min(CT, *t0 + per);
}

}  // namespace sv
