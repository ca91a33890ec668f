// Greedy MTP verify/accept (include/moe_accept.h) as one gfx950 launch.
//
// The verify and accept steps of "Support Step3.5/3.7 flash mtp3" (Overview,
// data-flow trace of one MTP step, steps 4 and 5): the greedy token of every
// verify row, the number of drafts that agree with it, the accepted list and
// the hidden-state row kept for the next round.
//
// The logits are the only large input (M rows of a whole vocabulary), read
// once.  Workgroup b takes columns [b*C, (b+1)*C) of every row; a thread
// reads four consecutive columns of four rows per pass (16-byte loads where
// the rows are 16-byte aligned) and keeps the best (key, column) of each
// row, with order-preserving integer keys so the comparison is exact.  The
// wave reduces with DPP, the four waves through LDS, and the workgroup's
// result per row goes to the workspace with write-through stores.  The last
// workgroup to arrive reduces each row's partials (one wave per row), runs
// the accept rule, copies verify row n_accepted to pending_h and returns
// the counter to zero.
#include <hip/hip_runtime.h>

#include "common.h"
#include "moe_accept.h"

namespace svr {
namespace {

constexpr int kColsPerPass = 4 * kBlock;  // columns a workgroup covers per pass
constexpr int kRowGroup = 4;              // rows a thread reads per pass
constexpr int kAcceptMaxBlocks = 1024;
constexpr uint32_t kNoCol = 0xFFFFFFFFu;

struct AcceptArgs {
  const float* logits;
  int64_t V;
  int64_t cols_per_block;
  int M, nblocks;
  const int32_t* drafts;
  const float* vh;  // verify_h, NULL: no hidden-state copy
  int hdim;
  int32_t* tokens;
  int32_t* accepted;
  int32_t* n_acc;
  float* pending;
  unsigned* ctr;
  uint64_t* part;  // [nblocks][M]: key << 32 | column
};

// (k, c) replaces (bk, bc) if its key is larger, or equal with a lower column.
__device__ __forceinline__ void better(uint32_t& bk, uint32_t& bc, uint32_t k, uint32_t c) {
  if (k > bk || (k == bk && c < bc)) {
    bk = k;
    bc = c;
  }
}

// Best (key, column) over the wave, in every lane.
__device__ __forceinline__ void wave_best(uint32_t& bk, uint32_t& bc) {
  const uint32_t k = wave_max_u32(bk);
  bc = wave_min_u32(bk == k ? bc : kNoCol);
  bk = k;
}

template <bool VEC>
__global__ __launch_bounds__(kBlock) void k_accept(AcceptArgs a) {
  __shared__ uint32_t s_k[kWavesPerBlock][kRowGroup], s_c[kWavesPerBlock][kRowGroup];
  __shared__ int s_last, s_n;
  __shared__ int32_t s_tok[MOE_ACCEPT_MAX_ROWS];
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
  const int64_t c_begin = (int64_t)blockIdx.x * a.cols_per_block;
  const int64_t c_end = min(c_begin + a.cols_per_block, a.V);

  for (int r0 = 0; r0 < a.M; r0 += kRowGroup) {
    uint32_t bk[kRowGroup], bc[kRowGroup];
#pragma unroll
    for (int i = 0; i < kRowGroup; ++i) {
      bk[i] = 0u;
      bc[i] = kNoCol;
    }
    for (int64_t c = c_begin + 4 * threadIdx.x; c < c_end; c += kColsPerPass) {
      float v[kRowGroup][4];
#pragma unroll
      for (int i = 0; i < kRowGroup; ++i) {
        // Rows past M re-read row M-1; their results are never stored.
        const float* p = a.logits + (int64_t)min(r0 + i, a.M - 1) * a.V + c;
        if (VEC && c + 3 < c_end) {
          const float4 q = ldf4(p);
          v[i][0] = q.x;
          v[i][1] = q.y;
          v[i][2] = q.z;
          v[i][3] = q.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[i][e] = (c + e < c_end) ? p[e] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < kRowGroup; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < c_end) better(bk[i], bc[i], order_key(v[i][e]), (uint32_t)(c + e));
    }
#pragma unroll
    for (int i = 0; i < kRowGroup; ++i) {
      wave_best(bk[i], bc[i]);
      if (lane == 0) {
        s_k[wv][i] = bk[i];
        s_c[wv][i] = bc[i];
      }
    }
    __syncthreads();
    if (threadIdx.x < kRowGroup && r0 + (int)threadIdx.x < a.M) {
      const int i = threadIdx.x;
      uint32_t k = s_k[0][i], cc = s_c[0][i];
#pragma unroll
      for (int w = 1; w < kWavesPerBlock; ++w) better(k, cc, s_k[w][i], s_c[w][i]);
      store_shared(a.part + (int64_t)blockIdx.x * a.M + r0 + i, ((uint64_t)k << 32) | cc);
    }
    __syncthreads();  // s_k / s_c are reused by the next row group
  }

  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive(a.ctr) == (unsigned)(a.nblocks - 1);
  __syncthreads();
  if (!s_last) return;

  // Last workgroup: every row's greedy token from the partials.
  for (int r = wv; r < a.M; r += kWavesPerBlock) {
    uint32_t k = 0u, cc = kNoCol;
    for (int b = lane; b < a.nblocks; b += kWave) {
      const uint64_t p = load_shared(a.part + (int64_t)b * a.M + r);
      better(k, cc, (uint32_t)(p >> 32), (uint32_t)p);
    }
    wave_best(k, cc);
    if (lane == 0) {
      s_tok[r] = (int32_t)cc;
      a.tokens[r] = (int32_t)cc;
    }
  }
  __syncthreads();
  // Accept rule: drafts are kept while row j's token equals draft j+1.
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < a.M - 1 && s_tok[n] == a.drafts[n]) ++n;
    s_n = n;
    *a.n_acc = n;
  }
  __syncthreads();
  const int n = s_n;
  for (int i = threadIdx.x; i < a.M; i += kBlock)
    a.accepted[i] = i < n ? a.drafts[i] : (i == n ? s_tok[n] : -1);
  if (a.vh) {
    const float* src = a.vh + (int64_t)n * a.hdim;
    for (int i = threadIdx.x; i < a.hdim; i += kBlock) a.pending[i] = src[i];
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr size_t kCounterLine = 256;

// Columns per workgroup: whole passes, at most kAcceptMaxBlocks workgroups.
int64_t cols_per_block(int64_t V) {
  const int64_t per = (int64_t)kColsPerPass * kAcceptMaxBlocks;
  return (int64_t)kColsPerPass * ((V + per - 1) / per);
}

size_t ws_bytes(int M, int64_t V) {
  const int64_t B = (V + cols_per_block(V) - 1) / cols_per_block(V);
  return kCounterLine + (((size_t)B * (size_t)M * 8 + 255) & ~(size_t)255);
}

}  // namespace
}  // namespace svr

using namespace svr;

extern "C" {

int32_t moe_accept_workspace_bytes(int32_t max_rows, int64_t vocab, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  if (max_rows < 1 || max_rows > MOE_ACCEPT_MAX_ROWS || vocab < 1 || vocab > MOE_ACCEPT_MAX_VOCAB)
    return MOE_ERR_SHAPE;
  *bytes = ws_bytes(max_rows, vocab);
  return MOE_OK;
}

int32_t moe_verify_accept(const float* logits, int32_t n_rows, int64_t vocab,
                          const int32_t* drafts, const float* verify_h, int32_t h_dim,
                          int32_t* tokens, int32_t* accepted, int32_t* n_accepted,
                          float* pending_h, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
  if (n_rows < 0 || n_rows > MOE_ACCEPT_MAX_ROWS || vocab < 1 || vocab > MOE_ACCEPT_MAX_VOCAB ||
      h_dim < 0)
    return MOE_ERR_SHAPE;
  if (n_rows == 0) return MOE_OK;
  if (!logits || !tokens || !accepted || !n_accepted || !workspace) return MOE_ERR_NULL;
  if (n_rows > 1 && !drafts) return MOE_ERR_NULL;
  if ((verify_h == nullptr) != (pending_h == nullptr)) return MOE_ERR_NULL;
  if (!verify_h && h_dim > 0) return MOE_ERR_SHAPE;
  if (workspace_bytes < ws_bytes(n_rows, vocab)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)workspace % 256) return MOE_ERR_ARG;
  if ((uintptr_t)logits % 4) return MOE_ERR_ARG;

  AcceptArgs a{};
  a.logits = logits;
  a.V = vocab;
  a.cols_per_block = cols_per_block(vocab);
  a.M = n_rows;
  a.nblocks = (int)((vocab + a.cols_per_block - 1) / a.cols_per_block);
  a.drafts = drafts;
  a.vh = verify_h;
  a.hdim = verify_h ? h_dim : 0;
  a.tokens = tokens;
  a.accepted = accepted;
  a.n_acc = n_accepted;
  a.pending = pending_h;
  a.ctr = (unsigned*)workspace;
  a.part = (uint64_t*)((uint8_t*)workspace + kCounterLine);
  const bool vec = (uintptr_t)logits % 16 == 0 && vocab % 4 == 0;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  if (vec)
    hipLaunchKernelGGL(k_accept<true>, dim3(a.nblocks), dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(k_accept<false>, dim3(a.nblocks), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"
