// S3/S4: init_routing and compute_expert_tokens ([Qwen3] "GMM enablement
// and routing optimisation"): per-expert histogram of the top-k ids, an
// exclusive prefix scan, and a stable counting-sort scatter of the pairs
// p = t*k + j by expert, plus the inverse permutation.
//
// One 8-bit digit (E <= 256) means one counting-sort pass.  Pairs are cut
// into chunks of RCHUNK; with more than one chunk a first kernel writes each
// chunk's histogram to the workspace.  The scatter kernel (one 1024-thread
// block per chunk, one pair per thread) turns the histograms into
// per-expert bases (global exclusive scan + the counts of earlier chunks)
// and places its chunk's pairs in order in one round: ranked inside a wave
// by matching the 8 id bits with ballots and across the block's 16 waves
// through per-wave counts in LDS.  No atomics touch global memory, so the
// result is deterministic.
//
// Up to RDIRECT chunks every scatter block sums the histograms it needs
// itself (chunks x (E+1) loads per block, no extra launch).  Beyond that a
// scan kernel first replaces each expert's column of chunk counts by its
// exclusive prefix over the chunks, in place, and writes the totals to one
// more row, so that each scatter block reads two rows: the work stays
// linear in the number of chunks instead of quadratic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int RCHUNK = 1024;
constexpr int RDIRECT = 64;

size_t route_workspace_bytes(int T, int k, int E) {
  const long long R = (long long)T * k;
  const long long nb = (R + RCHUNK - 1) / RCHUNK;
  if (nb <= 1) return 0;
  return (size_t)(nb + (nb > RDIRECT ? 1 : 0)) * (size_t)(E + 1) * sizeof(int32_t);
}

__global__ __launch_bounds__(256) void route_hist(const int32_t* __restrict__ ids, int R, int E,
                                                  int32_t* __restrict__ ws) {
  __shared__ int h[257];
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += 256) h[i] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * RCHUNK;
  const int p1 = min(R, p0 + RCHUNK);
  for (int p = p0 + tid; p < p1; p += 256) {
    const int e = ids[p];
    atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1);
  }
  __syncthreads();
  for (int i = tid; i <= E; i += 256) ws[(size_t)blockIdx.x * (E + 1) + i] = h[i];
}

// Column i (expert i, or E for the dropped pairs) of the chunk histograms:
// ws[c][i] becomes the count of i in chunks before c, ws[nb][i] the total.
// One block per column; thread t sums a contiguous run of chunks, a block
// scan gives each run its base, and the run is rewritten in order.
__global__ __launch_bounds__(256) void route_scan(int nb, int E, int32_t* __restrict__ ws) {
  __shared__ int wsum[4];
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t stride = (size_t)(E + 1);
  const int per = (nb + 255) / 256;
  const int c0 = min(nb, tid * per), c1 = min(nb, c0 + per);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += ws[(size_t)c * stride + i];
  const int incl = wave_incl_scan(sum);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int run = before + incl - sum;
  for (int c = c0; c < c1; ++c) {
    const size_t at = (size_t)c * stride + i;
    const int v = ws[at];
    ws[at] = run;
    run += v;
  }
  if (tid == 255) ws[(size_t)nb * stride + i] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

__global__ __launch_bounds__(1024) void route_scatter(const int32_t* __restrict__ ids, int R,
                                                      int E, int nb, const int32_t* __restrict__ ws,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_pair,
                                                      int32_t* __restrict__ pair_pos,
                                                      int32_t* __restrict__ dev_status) {
  __shared__ int tot[257];
  __shared__ int run[256];
  __shared__ int wsum[4];
  __shared__ int wcnt[16][256];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int p = b * RCHUNK + tid;  // one pair per thread
  const bool inrange = p < R;
  const int e = inrange ? ids[p] : -1;
  const bool ok = inrange && e >= 0 && e < E;

  // 1. per-expert totals and the counts of earlier chunks
  if (nb == 1) {
    for (int i = tid; i <= E; i += 1024) tot[i] = 0;
    __syncthreads();
    if (inrange) atomicAdd(&tot[ok ? e : E], 1);
    for (int i = tid; i < E; i += 1024) run[i] = 0;
  } else if (nb > RDIRECT) {
    // prefixes and totals from route_scan
    for (int i = tid; i <= E; i += 1024) {
      tot[i] = ws[(size_t)nb * (E + 1) + i];
      if (i < E) run[i] = ws[(size_t)b * (E + 1) + i];
    }
  } else {
    for (int i = tid; i <= E; i += 1024) {
      int sum = 0, pre = 0;
      for (int bb = 0; bb < nb; ++bb) {
        const int v = ws[(size_t)bb * (E + 1) + i];
        if (bb < b) pre += v;
        sum += v;
      }
      tot[i] = sum;
      if (i < E) run[i] = pre;
    }
  }
  // the rank counts of the placement below start at zero
  for (int i = tid; i < 16 * 256; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();

  // 2. exclusive scan of the totals over experts (E <= 256 = one per thread
  // of waves 0..3)
  int v = 0, incl = 0;
  if (tid < 256) {
    v = tid < E ? tot[tid] : 0;
    incl = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = incl;
  }
  // 3. stable placement of the chunk's pairs in one round: within a wave by
  // matching the 8 id bits with ballots, across the 16 waves through
  // per-wave counts in LDS
  unsigned long long match = __ballot(ok);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool on = ok && ((e >> bit) & 1);
    const unsigned long long bb = __ballot(on);
    match &= ((e >> bit) & 1) ? bb : ~bb;
  }
  const int rank = __popcll(match & ((1ull << lane) - 1ull));
  if (ok && rank == 0) wcnt[wave][e] = __popcll(match);
  __syncthreads();
  if (tid < E) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + incl - v;
    run[tid] += excl;
    if (b == 0) {
      counts[tid] = v;
      offsets[tid] = excl;
      if (tid == E - 1) offsets[E] = excl + v;
    }
  }
  if (b == 0 && tid == 0 && dev_status != nullptr) *dev_status = tot[E] > 0 ? 1 : 0;
  __syncthreads();
  if (ok) {
    int pos = run[e] + rank;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
    sorted_pair[pos] = p;
    pair_pos[p] = pos;
  } else if (inrange) {
    pair_pos[p] = -1;
  }
}

int launch_route(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_pos, int32_t* dev_status, int32_t* ws,
                 hipStream_t s) {
  const int R = T * k;
  const int nb = (R + RCHUNK - 1) / RCHUNK;
  if (nb > 1) hipLaunchKernelGGL(route_hist, dim3(nb), dim3(256), 0, s, ids, R, E, ws);
  if (nb > RDIRECT) hipLaunchKernelGGL(route_scan, dim3(E + 1), dim3(256), 0, s, nb, E, ws);
  hipLaunchKernelGGL(route_scatter, dim3(nb), dim3(1024), 0, s, ids, R, E, nb, ws, counts, offsets,
                     sorted_pair, pair_pos, dev_status);
  return launch_status();
}

}  // namespace moe
