// route.hip -- top-k routing and the token-by-expert permutation.
//
// experts4bit-qlora 0.1.0 sdist, _vendor/experts.py, Experts4bit.forward takes
// (top_k_index, top_k_weights) from a router outside the module and groups the
// routed (token, slot) pairs per expert with a one-hot mask and torch.where,
// paying a device-to-host sync for every expert. Here the grouping is a stable
// counting sort done entirely on the device:
//   1. histogram of expert ids per chunk of kPermChunk pairs,
//   2. per expert, exclusive scan of its chunk counts,
//   3. per chunk, one wavefront assigns each pair its sorted position
//      (expert offset + chunk base + rank among equal ids, lanes in pair order).
#include "device.h"
#include "kernels.h"
#include "route_dev.h"

namespace e4b {

// One wavefront per token (route_dev.h).
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int64_t T,
                                                    int E, int k, int32_t *__restrict__ idx,
                                                    float *__restrict__ wts) {
  __shared__ RouteLds s_route[4];
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token(logits, t, E, k, lane, idx, wts, nullptr, s_route[threadIdx.x >> 6]);
}

// hist[e * nchunks + c] = number of pairs of chunk c routed to expert e.
__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t *__restrict__ flat_idx,
                                                        int64_t P, int E, int64_t nchunks,
                                                        int32_t *__restrict__ hist) {
  __shared__ int32_t h[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t c = blockIdx.x;
  const int64_t p0 = c * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    const int64_t p = p0 + i;
    if (p < P) atomicAdd(&h[safe_expert(flat_idx[p], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[int64_t(e) * nchunks + c] = h[e];
}

// One workgroup per expert: chunk_base[e][c] = sum_{c' < c} hist[e][c'],
// counts[e] = total.
__global__ __launch_bounds__(256) void perm_scan_kernel(const int32_t *__restrict__ hist,
                                                        int64_t nchunks,
                                                        int32_t *__restrict__ chunk_base,
                                                        int32_t *__restrict__ counts) {
  __shared__ int32_t wsum[4];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int32_t *hrow = hist + int64_t(e) * nchunks;
  int32_t *brow = chunk_base + int64_t(e) * nchunks;
  int32_t carry = 0;
  for (int64_t c0 = 0; c0 < nchunks; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    const int32_t v = c < nchunks ? hrow[c] : 0;
    int32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t n = __shfl_up(incl, o);
      if (lane >= o) incl += n;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int32_t before = carry;
    for (int i = 0; i < wv; ++i) before += wsum[i];
    if (c < nchunks) brow[c] = before + incl - v;
    const int32_t total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    carry += total;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// One wavefront per chunk. Writes sorted_pair / pos_of_pair; workgroup 0 also
// writes offsets[E+1], tile_offsets[E+1] (m-tiles of kBM rows per expert) and
// the tile map (expert, segment start, first row, rows) of every m-tile, so a
// GEMM workgroup finds its tile with one load.
__global__ __launch_bounds__(64) void perm_scatter_kernel(
    const int32_t *__restrict__ flat_idx, int64_t P, int E, int nbits, int64_t nchunks,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ chunk_base,
    int32_t *__restrict__ sorted_pair, int32_t *__restrict__ pos_of_pair,
    int32_t *__restrict__ offsets, int32_t *__restrict__ tile_offsets,
    int4 *__restrict__ tile_map, int64_t m_tiles_bound) {
  __shared__ int32_t base[kMaxE];
  const int lane = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int64_t p0 = c * kPermChunk;
  // the chunk's expert ids, all loads issued before the scan below
  constexpr int kIt = kPermChunk / 64;
  int ids[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int64_t p = p0 + it * 64 + lane;
    ids[it] = p < P ? safe_expert(flat_idx[p], E) : 0;
  }
  // exclusive scan of counts (and of m-tiles) over experts, 64 at a time
  int32_t carry = 0, tcarry = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int32_t v = e < E ? counts[e] : 0;
    const int32_t tv = (v + kBM - 1) / kBM;
    int32_t incl = v, tincl = tv;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t n = __shfl_up(incl, o), tn = __shfl_up(tincl, o);
      if (lane >= o) {
        incl += n;
        tincl += tn;
      }
    }
    if (e < E) {
      const int32_t off = carry + incl - v;
      base[e] = off + chunk_base[int64_t(e) * nchunks + c];
      if (c == 0) {
        offsets[e] = off;
        const int32_t t0 = tcarry + tincl - tv;
        tile_offsets[e] = t0;
        for (int t = 0; t < tv; ++t)
          tile_map[t0 + t] = int4{e, off, t * kBM, min(kBM, v - t * kBM)};
      }
    }
    carry += __shfl(incl, 63);
    tcarry += __shfl(tincl, 63);
  }
  if (c == 0 && lane == 0) {
    offsets[E] = carry;
    tile_offsets[E] = tcarry;
  }
  // unused tile map entries are zeroed (no stale bytes in a saved buffer)
  if (c == 0)
    for (int64_t t = tcarry + lane; t < m_tiles_bound; t += 64) tile_map[t] = int4{0, 0, 0, 0};
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int64_t p = p0 + it * 64 + lane;
    const bool valid = p < P;
    const int e = ids[it];
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const int rank = __popcll(match & lt);
    const int32_t my_base = valid ? base[e] : 0;
    __syncthreads();
    if (valid) {
      const int32_t pos = my_base + rank;
      sorted_pair[pos] = int32_t(p);
      pos_of_pair[p] = pos;
      // the highest lane of each equal-id group advances that expert's base
      if ((match >> lane) == 1ull) base[e] = my_base + __popcll(match);
    }
    __syncthreads();
  }
}

hipError_t launch_route(const float *logits, int64_t T, int E, int k, int32_t *idx, float *w,
                        hipStream_t s, const e4b_kernel_events *ev) {
  if (T == 0) return hipSuccess;
  return launch_k(ev, E4B_K_ROUTE, route_kernel, dim3(uint32_t((T + 3) / 4)), dim3(256), s, logits,
                  T, E, k, idx, w);
}

PermView perm_in_workspace(const MoePlan &p, char *ws) {
  PermView v;
  v.offsets = reinterpret_cast<int32_t *>(ws + p.off_offsets);
  v.tile_offsets = reinterpret_cast<int32_t *>(ws + p.off_tile_offsets);
  v.tile_map = reinterpret_cast<int4 *>(ws + p.off_tile_map);
  v.sorted = reinterpret_cast<int32_t *>(ws + p.off_sorted);
  v.pos = reinterpret_cast<int32_t *>(ws + p.off_pos);
  return v;
}

PermView perm_in_saved(const MoePlan &p, char *saved) {
  PermView v;
  v.offsets = reinterpret_cast<int32_t *>(saved + p.sv_offsets);
  v.tile_offsets = reinterpret_cast<int32_t *>(saved + p.sv_tile_offsets);
  v.tile_map = reinterpret_cast<int4 *>(saved + p.sv_tile_map);
  v.sorted = reinterpret_cast<int32_t *>(saved + p.sv_sorted);
  v.pos = reinterpret_cast<int32_t *>(saved + p.sv_pos);
  return v;
}

hipError_t launch_permute(const MoePlan &p, const int32_t *idx, char *ws, const PermView &v,
                          hipStream_t s, const e4b_kernel_events *ev) {
  if (p.P == 0) return hipSuccess;
  int32_t *hist = reinterpret_cast<int32_t *>(ws + p.off_hist);
  int32_t *cbase = reinterpret_cast<int32_t *>(ws + p.off_chunk_base);
  int32_t *counts = reinterpret_cast<int32_t *>(ws + p.off_counts);
  const int E = int(p.E);
  // E4B_K_PERMUTE spans the three launches: start event on the first, stop on the last
  hipEvent_t e0 = ev ? ev->start[E4B_K_PERMUTE] : nullptr, e1 = ev ? ev->stop[E4B_K_PERMUTE] : nullptr;
  const bool timed = e0 && e1;
  if (timed)
    hipExtLaunchKernelGGL(perm_hist_kernel, dim3(uint32_t(p.nchunks)), dim3(256), 0, s, e0,
                          static_cast<hipEvent_t>(nullptr), 0, idx, p.P, E, p.nchunks, hist);
  else
    hipLaunchKernelGGL(perm_hist_kernel, dim3(uint32_t(p.nchunks)), dim3(256), 0, s, idx, p.P, E,
                       p.nchunks, hist);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(uint32_t(E)), dim3(256), 0, s, hist, p.nchunks, cbase,
                     counts);
  if (timed)
    hipExtLaunchKernelGGL(perm_scatter_kernel, dim3(uint32_t(p.nchunks)), dim3(64), 0, s,
                          static_cast<hipEvent_t>(nullptr), e1, 0, idx, p.P, E, p.nbits_e,
                          p.nchunks, static_cast<const int32_t *>(counts),
                          static_cast<const int32_t *>(cbase), v.sorted, v.pos, v.offsets,
                          v.tile_offsets, v.tile_map, p.m_tiles_bound);
  else
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(uint32_t(p.nchunks)), dim3(64), 0, s, idx, p.P, E,
                       p.nbits_e, p.nchunks, counts, cbase, v.sorted, v.pos, v.offsets,
                       v.tile_offsets, v.tile_map, p.m_tiles_bound);
  return hipGetLastError();
}

}  // namespace e4b
