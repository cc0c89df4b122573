// KV-cache compaction after acceptance: the accepted path's tree rows move
// down to follow the prefix, the rest of the draft tree is dropped.
//
// What is computed ("EAGLE / EAGLE-2" excerpts, modelers.csdn.net, sec. 1.3.2:
// the accepted tokens are kept for the next drafting round; "EAGLE (ICML
// 2024) close reading", edgeai1.github.io, sec. 5: after a rejection both the
// target's and the draft decoder's caches are cut back): for sequence b with
// n = accept_len[b] >= 0 accepted nodes, in every layer,
//   row L_b + i  <-  row L_b + accept_path[b][i],   i < n,
// rows counted from kv_offset[b]; the new prefix length is L_b + n. Because
// the packed tree puts parents before children ("LLM speculative decoding:
// EAGLE", jingming.pro, sec. 4.2), the rows of a root-down path in this
// order are the rows a causal decode of the accepted tokens would have
// appended.
//
// In place without a second buffer: a valid path is strictly increasing, so
// path[i] >= i. A row j written as destination j is read as a source only by
// an earlier index k < j (path[k] = j), and a thread that walks i upwards
// reads that source before it writes row j. Threads split the row by byte
// columns, so every thread owns its columns across all rows of a (sequence,
// layer) and no two threads touch the same bytes. Loads of up to 8 rows are
// issued before their stores, which keeps the same order argument per batch.
#include "sv_internal.h"

namespace sv {

struct CompactParams {
  char* cache;
  long long layer_stride;   // bytes between layers
  int row_bytes;
  int B, N;
  const int32_t* kv_offset;
  const int32_t* prefix_len;
  const int32_t* accept_len;
  const int32_t* accept_path;
  int32_t* new_prefix_len;
  int32_t* status;
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCompactThreads = 256;
constexpr int kCompactBatch = 8;

template <typename V>
__global__ __launch_bounds__(kCompactThreads) void k_compact_cache(CompactParams p) {
  const int b = blockIdx.y;
  const int layer = blockIdx.z;
  const int n = p.accept_len[b];
  const int L = p.prefix_len[b];
  const long long r0 = p.kv_offset[b];
  const long long r1 = p.kv_offset[b + 1];
  const int32_t* path = p.accept_path + (size_t)b * p.N;
  // every thread checks the same data and reaches the same verdict
  bool ok = n >= -1 && n <= p.N && L >= 0 && r0 >= 0 && r0 + L + p.N <= r1;
  if (ok) {
    int prev = -1;
    for (int i = 0; i < n; ++i) {
      const int j = path[i];
      if (j <= prev || j >= p.N) {
        ok = false;
        break;
      }
      prev = j;
    }
  }
  if (blockIdx.x == 0 && layer == 0 && threadIdx.x == 0) {
    p.new_prefix_len[b] = (ok && n > 0) ? L + n : L;
    if (p.status) p.status[b] = ok ? 0 : kSeqErrPath;
  }
  if (!ok || n <= 0) return;
  const int units = p.row_bytes / (int)sizeof(V);
  const int u = blockIdx.x * kCompactThreads + threadIdx.x;
  if (u >= units) return;
  char* base = p.cache + (long long)layer * p.layer_stride + (r0 + L) * p.row_bytes +
               (long long)u * sizeof(V);
  for (int i0 = 0; i0 < n; i0 += kCompactBatch) {
    V v[kCompactBatch];
    // past the end, re-read the last row (always valid) so the batch stays
    // in registers; only the stores are conditional
#pragma unroll
    for (int k = 0; k < kCompactBatch; ++k)
      v[k] = *(const V*)(base + (long long)path[min(i0 + k, n - 1)] * p.row_bytes);
#pragma unroll
    for (int k = 0; k < kCompactBatch; ++k)
      if (i0 + k < n) *(V*)(base + (long long)(i0 + k) * p.row_bytes) = v[k];
  }
}

hipError_t launch_compact_cache(void* cache, long long layer_stride, int n_layers, int row_bytes,
                                int B, int N, const int32_t* kv_offset,
                                const int32_t* prefix_len, const int32_t* accept_len,
                                const int32_t* accept_path, int32_t* new_prefix_len,
                                int32_t* status, bool vec16, hipStream_t s) {
  CompactParams p{(char*)cache, layer_stride, row_bytes, B, N, kv_offset, prefix_len,
                  accept_len, accept_path, new_prefix_len, status};
  const int units = row_bytes / (vec16 ? 16 : 4);
  const dim3 grid((units + kCompactThreads - 1) / kCompactThreads, B, n_layers);
  if (vec16)
    hipLaunchKernelGGL(k_compact_cache<u32x4_t>, grid, dim3(kCompactThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_compact_cache<uint32_t>, grid, dim3(kCompactThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
