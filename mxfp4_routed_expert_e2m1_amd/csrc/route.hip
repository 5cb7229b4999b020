// route.hip -- top-k routing and bit-exact stable expert grouping.
//
// Routing: gfx90a report §3.2 (256 routed experts, top-6 per token) and §5.3
// (membership ties broken by logical id, selected positions in a fixed
// order).  One wave per token: k rounds of a wave-wide arg-max over
// (logit desc, index asc); weights are fp32 sigmoid scores renormalised over
// the k picks.
//
// Grouping: gfx90a report §7.1 item 8 (the expert sorter groups assignments
// so each expert scans its packed weights once); the result is the stable
// counting sort by expert.  Decode-sized calls (one workgroup, top-k
// included): an assignment's position is its rank by (expert, index),
// counted over the few ids in LDS.  Larger calls: each wave counts its own
// contiguous range of assignments per expert, a scan gives every wave its
// base per expert, and each wave scatters its range in order, a lane's
// destination being the running base + its rank among earlier lanes of its
// wave with the same expert (from ballots).  No atomic decides an order, so
// the permutation is unique and bit-exact.
#include <float.h>

#include "common.h"

namespace moe {

constexpr int kMaxExperts = 512;  // keeps the grouping LDS under 64 KiB
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t ld_l, int rows, int n_experts,
                                                         int top_k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int row = (int)(((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (row >= rows) return;  // whole wave exits together
  int id;
  float wt;
  topk_row<PER_LANE>(logits + (int64_t)row * ld_l, n_experts, top_k, &id, &wt);
  const int lane = lane_id();
  if (lane < top_k) {
    ids[(int64_t)row * top_k + lane] = id;
    w[(int64_t)row * top_k + lane] = wt;
  }
}

// Grouping of the ids of any number of rows (after route_topk_kernel).
constexpr int kFusedMaxAssign = kGroupWaves * MOE_MAX_TOP_K;

// Each wave owns a contiguous range of assignment indices (a multiple of 64)
// and walks it in 64-wide pieces, kGroupWindow pieces per round trip of id
// loads.  Pass 1 counts each wave's assignments per expert (LDS atomic adds
// into the wave's own row: a count does not depend on their order); one scan
// turns the counts into each wave's base per expert (the expert's offset
// plus the counts of the earlier waves); pass 2 scatters each wave's range in
// order, a lane's position being its wave's running base for the expert plus
// its rank among the lower lanes with the same expert.  The running bases
// are private to a wave, so the scatter needs no workgroup barrier.
constexpr int kGroupWindow = 16;

// Per lane: rank among lower lanes holding the same (valid) expert, and that
// expert's count in the wave.
__device__ inline void wave_match(int e, bool valid, int nbits, uint64_t lt_mask, int& rank,
                                  int& cnt) {
  uint64_t same = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool b = valid && ((e >> bit) & 1);
    const uint64_t m = __ballot(b);
    same &= ((e >> bit) & 1) ? m : ~m;
  }
  rank = __popcll(same & lt_mask);
  cnt = __popcll(same);
}

__global__ __launch_bounds__(kGroupThreads) void group_kernel(
    const int32_t* __restrict__ ids_g, int n_assign, int n_experts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted) {
  extern __shared__ int wbase[];  // [kGroupWaves][n_experts]: counts, then running bases
  __shared__ int wave_tot[kGroupWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int nbits = 0;
  while ((1 << nbits) < n_experts) ++nbits;
  // this wave's range [r0, r1) of assignments, in 64-wide pieces
  const int per_wave = (n_assign + kGroupWaves * 64 - 1) / (kGroupWaves * 64) * 64;
  const int r0 = min(wave * per_wave, n_assign), r1 = min(r0 + per_wave, n_assign);
  int* my = wbase + wave * n_experts;

  for (int e = tid; e < kGroupWaves * n_experts; e += kGroupThreads) wbase[e] = 0;
  __syncthreads();
  // pass 1: this wave's count per expert
  for (int w0 = r0; w0 < r1; w0 += kGroupWindow * 64) {
    int ev[kGroupWindow];
#pragma unroll
    for (int k = 0; k < kGroupWindow; ++k) {
      const int a = w0 + 64 * k + lane;
      ev[k] = a < r1 ? ids_g[a] : -1;
    }
#pragma unroll
    for (int k = 0; k < kGroupWindow; ++k)
      if (ev[k] >= 0) atomicAdd(&my[ev[k]], 1);
  }
  __syncthreads();

  // counts, offsets (exclusive scan over experts), and each wave's base per
  // expert (n_experts <= kGroupThreads: one expert per thread)
  int c = 0;
  if (tid < n_experts) {
    for (int w2 = 0; w2 < kGroupWaves; ++w2) c += wbase[w2 * n_experts + tid];
  }
  const int incl = wave_incl_scan(c);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w2 = 0; w2 < wave; ++w2) base += wave_tot[w2];
  const int excl = base + incl - c;
  if (tid < n_experts) {
    counts[tid] = c;
    offsets[tid] = excl;
    int run = excl;
    for (int w2 = 0; w2 < kGroupWaves; ++w2) {
      const int t = wbase[w2 * n_experts + tid];
      wbase[w2 * n_experts + tid] = run;
      run += t;
    }
  }
  int n_valid = 0;
  for (int w2 = 0; w2 < kGroupWaves; ++w2) n_valid += wave_tot[w2];
  if (tid == 0) offsets[n_experts] = n_valid;
  __syncthreads();

  // pass 2: scatter this wave's range in index order
  for (int w0 = r0; w0 < r1; w0 += kGroupWindow * 64) {
    int ev[kGroupWindow];
#pragma unroll
    for (int k = 0; k < kGroupWindow; ++k) {
      const int a = w0 + 64 * k + lane;
      ev[k] = a < r1 ? ids_g[a] : -1;
    }
#pragma unroll
    for (int k = 0; k < kGroupWindow; ++k) {
      if (w0 + 64 * k >= r1) break;  // wave-uniform
      const int e = ev[k];
      const bool valid = e >= 0;
      int rank, cnt;
      wave_match(e, valid, nbits, lt_mask, rank, cnt);
      const int pos = valid ? my[e] + rank : 0;
      if (valid) sorted[pos] = w0 + 64 * k + lane;
      // every lane has read the bases before the leaders move them on
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == 0) my[e] += cnt;
      __builtin_amdgcn_wave_barrier();
    }
  }
  for (int p = n_valid + tid; p < n_assign; p += kGroupThreads) sorted[p] = -1;
}

// Decode-sized rows (<= kGroupWaves, so at most kFusedMaxAssign
// assignments): top-k of each row by one wave; then every assignment's
// sorted position is its rank by the key expert * 256 + index -- the stable
// counting sort's result -- and every expert's count and offset are counts
// of keys below two bounds, one compare per key over the (few) keys in LDS.
// No histogram atomics, no scan phases.
struct RouteArgs {
  const float* logits;
  int64_t ld_l;
  int rows, top_k, n_experts;
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted;
};

// The whole decode route + group, run by one workgroup of kGroupThreads.
template <int PER_LANE>
__device__ inline void route_decode_wg(const RouteArgs& p) {
  const float* __restrict__ logits = p.logits;
  const int64_t ld_l = p.ld_l;
  const int rows = p.rows, top_k = p.top_k, n_experts = p.n_experts;
  int32_t* __restrict__ ids_g = p.ids;
  float* __restrict__ w_g = p.w;
  int32_t* __restrict__ counts = p.counts;
  int32_t* __restrict__ offsets = p.offsets;
  int32_t* __restrict__ sorted = p.sorted;
  __shared__ int ids_l[kFusedMaxAssign];
  __shared__ __align__(16) int keys_l[kFusedMaxAssign + 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_assign = rows * top_k;
  if (wave < rows) {
    int id;
    float wt;
    topk_row<PER_LANE>(logits + (int64_t)wave * ld_l, n_experts, top_k, &id, &wt);
    if (lane < top_k) {
      ids_g[wave * top_k + lane] = id;
      w_g[wave * top_k + lane] = wt;
      ids_l[wave * top_k + lane] = id;
    }
  }
  __syncthreads();
  // one sortable key per assignment: expert * 256 + index (index < 256),
  // sentinels and padding above every key
  constexpr int kNone = 0x7FFFFFFF;
  const int n16 = (n_assign + 15) >> 4;
  for (int b = tid; b < 16 * n16; b += kGroupThreads) {
    const int e = b < n_assign ? ids_l[b] : -1;
    keys_l[b] = e >= 0 ? e * 256 + b : kNone;
  }
  __syncthreads();
  // the keys, 16 at a time (four LDS reads in flight per step)
  auto scan = [&](auto&& f) {
    for (int b16 = 0; b16 < n16; ++b16) {
      int4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *(const int4*)&keys_l[16 * b16 + 4 * u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        f(v[u].x);
        f(v[u].y);
        f(v[u].z);
        f(v[u].w);
      }
    }
  };
  // sorted position of assignment tid: the keys below its own; positions
  // past the valid ones get -1
  if (tid < n_assign) {
    const int key = keys_l[tid];
    int pos = 0, n_valid = 0;
    scan([&](int k) {
      pos += k < key ? 1 : 0;
      n_valid += k != kNone ? 1 : 0;
    });
    if (key != kNone) sorted[pos] = tid;
    if (tid >= n_valid) sorted[tid] = -1;
  }
  // count and first position of every expert (offsets[n_experts]: all valid)
  for (int e = tid; e <= n_experts; e += kGroupThreads) {
    const int lo = e * 256, hi = e < n_experts ? lo + 256 : kNone;
    int below = 0, upto = 0;
    scan([&](int k) {
      below += k < lo ? 1 : 0;
      upto += k < hi ? 1 : 0;
    });
    if (e < n_experts) counts[e] = upto - below;
    offsets[e] = below;
  }
}

template <int PER_LANE>
__global__ __launch_bounds__(kGroupThreads) void route_decode_kernel(RouteArgs p) {
  route_decode_wg<PER_LANE>(p);
}

struct QuantArgs {
  const float* x;
  int64_t ld_x;
  int rows, cols;
  int8_t* q;
  int64_t ld_q;
  float* s;
  int64_t ld_s;
};

// A decode step's two independent inputs in one launch: workgroup 0 routes
// and groups the rows; workgroups 1.. quantise the activations (the same
// per-thread quantiser as moe_quant_act_q8, so the codes are the same bits).
template <int PER_LANE>
__global__ __launch_bounds__(kGroupThreads) void prep_decode_kernel(QuantArgs qa, RouteArgs ra) {
  if (blockIdx.x == 0) {
    route_decode_wg<PER_LANE>(ra);
  } else {
    quant_q8_thread((int64_t)(blockIdx.x - 1) * kGroupThreads + threadIdx.x, qa.x, qa.ld_x,
                    qa.rows, qa.cols, qa.q, qa.ld_q, qa.s, qa.ld_s);
  }
}

int route_args_check(const float* logits, int64_t ld_l, int rows, int n_experts,
                            int top_k, const int32_t* ids, const float* w, const int32_t* counts,
                            const int32_t* offsets, const int32_t* sorted) {
  if (rows < 0) return MOE_ERR_INVALID_ARG;
  if (n_experts < 1 || n_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (top_k < 1 || top_k > n_experts || top_k > MOE_MAX_TOP_K) return MOE_ERR_SHAPE;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!logits || !ids || !w || !sorted)) return MOE_ERR_INVALID_ARG;
  if ((int64_t)rows * top_k > (1 << 24)) return MOE_ERR_SHAPE;
  if (rows > 0 && ld_l < n_experts) return MOE_ERR_STRIDE;
  if (!aligned(counts, 4) || !aligned(offsets, 4) || (rows > 0 && (!aligned(logits, 4) ||
      !aligned(ids, 4) || !aligned(w, 4) || !aligned(sorted, 4))))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route_group(const float* logits, int64_t ld_l, int rows, int n_experts,
                               int top_k, int32_t* ids, float* w, int32_t* counts,
                               int32_t* offsets, int32_t* sorted, void* stream) {
  const int rc = route_args_check(logits, ld_l, rows, n_experts, top_k, ids, w, counts, offsets,
                                  sorted);
  if (rc != MOE_OK) return rc;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  hipStream_t s = (hipStream_t)stream;
  const int per_lane = (n_experts + 63) / 64;
  const size_t lds = sizeof(int) * (size_t)kGroupWaves * (size_t)n_experts;
  const int n_assign = rows * top_k;
  if (rows > 0 && rows <= kGroupWaves) {
    // decode-sized: top-k and grouping in one workgroup, one launch
    const RouteArgs ra{logits, ld_l, rows, top_k, n_experts, ids, w, counts, offsets, sorted};
    if (per_lane <= 4)
      hipLaunchKernelGGL(route_decode_kernel<4>, dim3(1), dim3(kGroupThreads), 0, s, ra);
    else
      hipLaunchKernelGGL(route_decode_kernel<8>, dim3(1), dim3(kGroupThreads), 0, s, ra);
    return launch_status();
  }
  if (rows > 0) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (per_lane <= 4)
      hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, ld_l, rows, n_experts,
                         top_k, ids, w);
    else
      hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, ld_l, rows,
                         n_experts, top_k, ids, w);
  }
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupThreads), lds, s, ids, n_assign,
                     n_experts, counts, offsets, sorted);
  return launch_status();
}

extern "C" int moe_decode_prep(const float* x, int64_t ld_x, int cols, int8_t* q, int64_t ld_q,
                               float* scales, int64_t ld_s, const float* logits, int64_t ld_l,
                               int rows, int n_experts, int top_k, int32_t* ids, float* w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted, void* stream) {
  if (rows < 1 || rows > MOE_MAX_DECODE_ROWS || rows > kGroupWaves) return MOE_ERR_SHAPE;
  int rc = quant_args_check(x, ld_x, rows, cols, q, ld_q, scales, ld_s);
  if (rc != MOE_OK) return rc;
  rc = route_args_check(logits, ld_l, rows, n_experts, top_k, ids, w, counts, offsets, sorted);
  if (rc != MOE_OK) return rc;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  const QuantArgs qa{x, ld_x, rows, cols, q, ld_q, scales, ld_s};
  const RouteArgs ra{logits, ld_l, rows, top_k, n_experts, ids, w, counts, offsets, sorted};
  const int64_t q_threads = (int64_t)rows * (cols / 8);
  const dim3 grid((unsigned)(1 + (q_threads + kGroupThreads - 1) / kGroupThreads));
  hipStream_t s = (hipStream_t)stream;
  if ((n_experts + 63) / 64 <= 4)
    hipLaunchKernelGGL(prep_decode_kernel<4>, grid, dim3(kGroupThreads), 0, s, qa, ra);
  else
    hipLaunchKernelGGL(prep_decode_kernel<8>, grid, dim3(kGroupThreads), 0, s, qa, ra);
  return launch_status();
}
