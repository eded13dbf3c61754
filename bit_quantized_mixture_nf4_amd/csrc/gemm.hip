// gemm.hip -- grouped GEMM over routed pairs with the 4-bit weight dequantized
// on the fly (bf16 MFMA, fp32 accumulation).
//
// One launch covers every expert (the grouped-nf4-gemm design the 0.31.1
// project page describes: one launch over the packed stacks, decode in the
// kernel, fp32 accumulation). Rows of a tile are routed pairs of one expert in
// sorted order; the tile schedule is read from device-side offsets, so the
// host never synchronizes.
//
// Operand modes
//   A_GATHER : A[m] = src[token(sorted_pair[row])]   (x or grad_y, [T, lda])
//   A_DIRECT : A[m] = src[row]                       (a or dGU, sorted rows)
//   B_NT     : B[n][k] = W[n][k]   weight rows are output columns (forward)
//   B_NN     : B[n][k] = W[k][n]   weight rows are the reduction (dgrad:
//              grad_output @ W, bitsandbytes PR #1965 recompute bullet)
// Epilogues
//   EPI_SWIGLU  : columns are gate/up pairs; a = silu(g) * u -> bf16, and the
//                 bf16 g, u are optionally stored for the backward
//                 (0.1.0 sdist, Experts4bit.forward: chunk into gate | up).
//   EPI_STORE   : bf16 store.
//   EPI_DSWIGLU : dgrad of act(gate) * up scaled by the routing weight, plus
//                 this tile's share of d y / d routing weight.
//
// Tile: kBM x kBN x kBK = 256 x 256 x 64 (one quantization block per K-step),
// 256 threads = 4 waves in 2 x 2, each wave 128 x 128 = 4 x 4 MFMA 32x32x16
// tiles. A and the dequantized B are staged in double-buffered LDS; B is
// dequantized once per workgroup (codebook in LDS, fp32 multiply by the block
// absmax, round-to-nearest-even bf16), i.e. exactly the bf16 view that
// e4b_dequantize_nf4 returns.
#include "device.h"
#include "kernels.h"

namespace e4b {

enum { A_GATHER = 0, A_DIRECT = 1 };
enum { B_NT = 0, B_NN = 1 };
enum { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_DSWIGLU = 2 };



constexpr int kThreads = 256;
constexpr int kLds = kBK + 8;  // padded row (bf16 elements): 144 bytes, conflict-free b128 access

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <int AMODE, int BMODE, int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLds];
  __shared__ float sCode[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile -> (expert, m-tile, n-tile) ----
  const uint32_t L = xcd_remap(blockIdx.x, g.grid);
  const int mt = int(L / uint32_t(g.n_tiles));
  const int nt = int(L % uint32_t(g.n_tiles));
  if (mt >= g.tile_offsets[g.E]) return;
  int lo = 0, hi = g.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.tile_offsets[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int seg = g.offsets[e];
  const int row0 = (mt - g.tile_offsets[e]) * kBM;
  const int valid_rows = min(kBM, g.offsets[e + 1] - seg - row0);

  if (tid < 16) sCode[tid] = codebook_value(g.cb, tid);

  // ---- A source rows: thread handles column chunk (tid & 7), rows (tid >> 3) + 32 i ----
  const int a_cc = tid & 7;
  uint32_t a_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    uint32_t off = 0xFFFFFFFFu;
    if (r < valid_rows) {
      const int srow = seg + row0 + r;
      const int src = AMODE == A_GATHER ? g.sorted_pair[srow] / g.topk : srow;
      off = uint32_t(src) * uint32_t(g.lda) + uint32_t(a_cc * 8);
    }
    a_off[i] = off;
  }

  // ---- B source ----
  const uint8_t *wp = g.Wp + int64_t(e) * g.w_e_bytes;
  const float *wa = g.Wa + int64_t(e) * g.w_e_blocks;
  const int row_bytes = g.w_in >> 1, row_blocks = g.w_in >> 6;
  // B_NT: this thread owns tile column tid (one weight row)
  int b_row = 0;
  bool b_valid = false;
  if (BMODE == B_NT) {
    if (EPI == EPI_SWIGLU) {
      const int c = tid;
      const int cw = c >> 7, j = (c & 127) >> 5, ll = c & 31;
      const int pair = nt * (kBN / 2) + cw * 64 + (j & 1) * 32 + ll;
      b_valid = pair < g.I;
      b_row = pair + (j >= 2 ? g.I : 0);
    } else {
      b_row = nt * kBN + tid;
      b_valid = b_row < g.N;
    }
  }
  // B_NN: this thread owns an 8 (k) x 8 (n) patch: n group cg, k group kg
  const int b_cg = tid >> 3, b_kg = tid & 7;
  const int b_n = nt * kBN + b_cg * 8;
  if (BMODE == B_NN) b_valid = b_n < g.N;

  u32x4 ra[8];
  u32x4 rb[2];
  uint32_t rbn[8];
  float ram[8];

  auto load = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (a_off[i] != 0xFFFFFFFFu)
        ra[i] = *reinterpret_cast<const u32x4 *>(g.A + a_off[i] + uint32_t(ks * kBK));
      else
        ra[i] = u32x4{0, 0, 0, 0};
    }
    if (BMODE == B_NT) {
      if (b_valid) {
        const u32x4 *src =
            reinterpret_cast<const u32x4 *>(wp + int64_t(b_row) * row_bytes + ks * (kBK / 2));
        rb[0] = src[0];
        rb[1] = src[1];
        ram[0] = wa[int64_t(b_row) * row_blocks + ks];
      } else {
        rb[0] = rb[1] = u32x4{0, 0, 0, 0};
        ram[0] = 0.0f;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t k = int64_t(ks) * kBK + b_kg * 8 + r;
        if (b_valid) {
          rbn[r] = *reinterpret_cast<const uint32_t *>(wp + k * row_bytes + (b_n >> 1));
          ram[r] = wa[k * row_blocks + (b_n >> 6)];
        } else {
          rbn[r] = 0;
          ram[r] = 0.0f;
        }
      }
    }
  };

  auto store = [&](int buf) {
    uint16_t *a_dst = sA[buf];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4 *>(a_dst + r * kLds + a_cc * 8) = ra[i];
    }
    uint16_t *b_dst = sB[buf];
    if (BMODE == B_NT) {
      const float am = ram[0];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t w = rb[d >> 2][d & 3];
        float v[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          v[2 * b] = __fmul_rn(sCode[(w >> (8 * b + 4)) & 15u], am);
          v[2 * b + 1] = __fmul_rn(sCode[(w >> (8 * b)) & 15u], am);
        }
        *reinterpret_cast<u32x4 *>(b_dst + tid * kLds + d * 8) =
            u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7])};
      }
    } else {
      float v[8][8];  // [k row r][n col c]
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t w = rbn[r];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          v[r][2 * b] = __fmul_rn(sCode[(w >> (8 * b + 4)) & 15u], ram[r]);
          v[r][2 * b + 1] = __fmul_rn(sCode[(w >> (8 * b)) & 15u], ram[r]);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        *reinterpret_cast<u32x4 *>(b_dst + (b_cg * 8 + c) * kLds + b_kg * 8) =
            u32x4{pack_bf16x2(v[0][c], v[1][c]), pack_bf16x2(v[2][c], v[3][c]),
                  pack_bf16x2(v[4][c], v[5][c]), pack_bf16x2(v[6][c], v[7][c])};
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // number of 32-row MFMA tiles of this wave that hold valid rows
  const int mi_valid = max(0, min(4, (valid_rows - wm * 128 + 31) >> 5));

  const int nK = g.K / kBK;
  __syncthreads();  // sCode visible
  load(0);
  store(0);
  if (nK > 1) load(1);
  __syncthreads();

  for (int ks = 0; ks < nK; ++ks) {
    const int cur = ks & 1;
    const uint16_t *a_src = sA[cur] + (wm * 128 + (lane & 31)) * kLds + (lane >> 5) * 8;
    const uint16_t *b_src = sB[cur] + (wn * 128 + (lane & 31)) * kLds + (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8 *>(a_src + i * 32 * kLds + kk * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8 *>(b_src + j * 32 * kLds + kk * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < mi_valid) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (ks + 1 < nK) store(cur ^ 1);
    if (ks + 2 < nK) load(ks + 2);
    __syncthreads();
  }

  // ---- epilogue ----
  // acc[i][j][r]: row = wm*128 + i*32 + 8*(r/4) + 4*(lane/32) + r%4,
  //               col = wn*128 + j*32 + lane%32
  const int lrow_base = wm * 128 + 4 * (lane >> 5);
  if (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = lrow_base + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row < valid_rows) {
          const int64_t grow = seg + row0 + row;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = nt * kBN + wn * 128 + j * 32 + (lane & 31);
            if (col < g.N) g.C[grow * g.ldc + col] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
  } else if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = lrow_base + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row < valid_rows) {
          const int64_t grow = seg + row0 + row;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int pair = nt * (kBN / 2) + wn * 64 + jj * 32 + (lane & 31);
            if (pair < g.I) {
              const float gv = acc[i][jj][r], uv = acc[i][jj + 2][r];
              const float a = gv * sigmoidf_(gv) * uv;
              if (g.C) g.C[grow * g.ldc + pair] = f32_to_bf16(a);
              if (g.GU) {
                g.GU[grow * (2 * g.I) + pair] = f32_to_bf16(gv);
                g.GU[grow * (2 * g.I) + g.I + pair] = f32_to_bf16(uv);
              }
            }
          }
        }
      }
    }
  } else {  // EPI_DSWIGLU
    float *red = reinterpret_cast<float *>(sA[0]);  // [2][kBM] partial row sums
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = lrow_base + i * 32 + 8 * (r >> 2) + (r & 3);
        float part = 0.0f;
        if (row < valid_rows) {
          const int64_t grow = seg + row0 + row;
          const float wr = g.topk_w[g.sorted_pair[grow]];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = nt * kBN + wn * 128 + j * 32 + (lane & 31);
            if (n < g.N) {
              const float gv = bf16_to_f32(g.GU[grow * (2 * g.I) + n]);
              const float uv = bf16_to_f32(g.GU[grow * (2 * g.I) + g.I + n]);
              const float s = sigmoidf_(gv);
              const float silu = gv * s;
              const float G2 = acc[i][j][r];
              part += G2 * (silu * uv);
              const float ga = wr * G2;
              const float dg = ga * uv * s * (1.0f + gv * (1.0f - s));
              const float du = ga * silu;
              g.C[grow * g.ldc + n] = f32_to_bf16(dg);
              g.C[grow * g.ldc + g.I + n] = f32_to_bf16(du);
            }
          }
        }
        // sum over the 32 columns held by this half-wave (fixed butterfly order)
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) part += __shfl_xor(part, o);
        if ((lane & 31) == 0) red[wn * kBM + i * 32 + 8 * (r >> 2) + (r & 3) + 4 * (lane >> 5) + wm * 128] = part;
      }
    }
    __syncthreads();
    if (tid < valid_rows) {
      const int64_t grow = seg + row0 + tid;
      g.partial[grow * g.n_tiles + nt] = red[tid] + red[kBM + tid];
    }
  }
}

hipError_t launch_grouped_gemm(GemmVariant v, const GemmArgs &a, hipStream_t s) {
  if (a.grid == 0) return hipSuccess;
  const dim3 grid(a.grid), block(kThreads);
  timer_before(int(v), s);
  switch (v) {
    case GEMM_GATE_UP_FWD:
      hipLaunchKernelGGL((grouped_gemm_kernel<A_GATHER, B_NT, EPI_SWIGLU>), grid, block, 0, s, a);
      break;
    case GEMM_DOWN_FWD:
      hipLaunchKernelGGL((grouped_gemm_kernel<A_DIRECT, B_NT, EPI_STORE>), grid, block, 0, s, a);
      break;
    case GEMM_DOWN_DGRAD:
      hipLaunchKernelGGL((grouped_gemm_kernel<A_GATHER, B_NN, EPI_DSWIGLU>), grid, block, 0, s, a);
      break;
    case GEMM_GATE_UP_DGRAD:
      hipLaunchKernelGGL((grouped_gemm_kernel<A_DIRECT, B_NN, EPI_STORE>), grid, block, 0, s, a);
      break;
  }
  const hipError_t err = hipGetLastError();
  timer_after(int(v), s);
  return err;
}

}  // namespace e4b
