// mx.hip -- the MX forward: MXFP4 expert weights against MXFP8 activations on
// gfx950's block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The 0.31.1 project page lists MXFP4 experts (gpt-oss) and a native MXFP4
// row; the formats are the OCP Microscaling Formats (MX) v1.0 ones: E2M1
// weights and E4M3 activations, each with an E8M0 scale per 32 elements along
// the reduction. The activations are converted per row (the pages do not
// describe them): x by mx8_rows_kernel before gate_up, a = bf16(silu(g) * u)
// inside the gate_up epilogue, which writes it only as MXFP8 rows for down.
//
// Operand layout of the instruction (cbsz = 4: A is E2M1, blgp = 0: B is E4M3),
// established with a probe kernel:
//   A (weights, 16 bytes of a v8i32): lane (row i = l % 32, half h = l / 32)
//     holds k = 32 h + n in nibble n, low nibble first;
//   B (activations, 32 bytes): lane (column j = l % 32, half h) holds
//     k = 32 (b / 16) + 16 h + b % 16 in byte b;
//   scales: lane (i or j, half h) supplies the E8M0 byte of k-block h;
//   D: the usual 32x32 f32 layout (lane l, register r: row 8 (r / 4) +
//     4 (l / 32) + r % 4, column l % 32).
// The weights store element 2m in the high nibble of byte m, so the
// instruction's k pairs element k ^ 1 of a row with activation k; the
// activation rows are therefore written with the two bytes of every element
// pair swapped, and the products pair up correctly without any shuffle.
#include "device.h"
#include "kernels.h"

namespace e4b {

typedef int i32x8 __attribute__((ext_vector_type(8)));
enum { MX_GATHER = 0, MX_DIRECT = 1 };  // activation rows: by token / by sorted pair
enum { MX_SWIGLU = 0, MX_STORE = 1 };   // epilogue

// ---- MXFP8 conversion: E4M3 codes against a shared E8M0 exponent ----
// shared = floor(log2(amax)) - 8 (the frexp exponent, exact), clamped to
// [-127, 127]. For y = |v| * 2^-shared, binade e = max(floor(log2 y), -6)
// (the subnormals share the lowest; y = 0 takes it too) and n = y / 2^(e-3)
// rounded to the nearest integer, ties to even (exact: power-of-two scalings
// and rint). The code is 8 (e + 7) + (n - 8): n in [8, 16] on a normal binade,
// where n = 16 carries into the next binade's mantissa 0, and n in [0, 8] on
// the subnormal one (codes 0..8). Saturation is the clamp to 0x7E (448): every
// y at or above the 448 / 480 midpoint lands on 0x7F or beyond.
__device__ __forceinline__ int mx8_shared(float amax) {
  return amax == 0.0f ? -127 : min(127, max(-127, __builtin_amdgcn_frexp_expf(amax) - 1 - 8));
}

__device__ __forceinline__ uint32_t e4m3_code(float v, int sh) {
  const float y = fabsf(ldexpf(v, -sh));
  const int e = y == 0.0f ? -6 : max(__builtin_amdgcn_frexp_expf(y) - 1, -6);
  const int n = int(rintf(ldexpf(y, 3 - e)));
  const uint32_t c = uint32_t(min(8 * e + 48 + n, 0x7E));
  return c | (signbit(v) ? 0x80u : 0u);
}

__global__ __launch_bounds__(256) void mx8_rows_kernel(const uint16_t *__restrict__ x,
                                                       int64_t nblocks,
                                                       uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales) {
  const int64_t blk = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + blk * kMxBlock);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 q = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_lo(q[j]);
      v[8 * i + 2 * j + 1] = bf16_hi(q[j]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int sh = mx8_shared(amax);
  u32x4 o[2];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    // bytes of element pair (2p, 2p + 1) stored swapped: element 2p + 1 first
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= e4m3_code(v[4 * d + (b ^ 1)], sh) << (8 * b);
    o[d >> 2][d & 3] = word;
  }
  u32x4 *dst = reinterpret_cast<u32x4 *>(codes + blk * kMxBlock);
  dst[0] = o[0];
  dst[1] = o[1];
  scales[blk] = uint8_t(sh + 127);
}

// ---- grouped GEMM on the block-scaled MFMA ----
// Tile 256 (pairs) x 256 (columns) x 128 (K-step: four MX blocks), 8 waves:
// 4 along M x 2 along N, each 64 x 128 (2 x 4 instructions per 64-deep half
// K-step). One workgroup per CU, two LDS stages; the two waves of a SIMD run
// a K-step's halves in opposite order, as in the 4-bit kernel. Staging is a
// plain copy: weights 16 KB, activations 32 KB and 2 KB of scales per step.
constexpr int kMxK = 128;
constexpr int kMxW = kMxK / 2 + 16;  // weight tile row stride (bytes): 64 + pad
constexpr int kMxA = kMxK + 16;      // activation tile row stride (bytes): 128 + pad

template <int AMODE, int EPI>
__global__ __launch_bounds__(512, 1) void mx_gemm_kernel(MxGemmArgs g) {
  constexpr int kThreads = 512, kBN = 256;
  __shared__ __attribute__((aligned(16))) uint8_t sW[2][kBN * kMxW];
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * kMxA];
  __shared__ __attribute__((aligned(16))) uint32_t sWs[2][kBN];  // 4 scale bytes per row
  __shared__ __attribute__((aligned(16))) uint32_t sAs[2][kBM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // tile -> (expert, m-tile, n-tile): the real tiles split evenly over the XCDs
  const int n_mt = g.tile_offsets[g.E];
  const uint32_t W = uint32_t(n_mt) * uint32_t(g.n_tiles);
  const uint32_t per_xcd = (W + 7) / 8, xi = blockIdx.x / 8;
  const uint32_t L = (blockIdx.x % 8) * per_xcd + xi;
  if (xi >= per_xcd || L >= W) return;
  const int mt = int(L / uint32_t(g.n_tiles)), nt = int(L % uint32_t(g.n_tiles));
  const int4 tm = g.tile_map[mt];
  const int e = tm.x, seg = tm.y, row0 = tm.z, valid_rows = tm.w;

  // activation rows: thread owns 16-byte chunk (tid & 7) of rows tid / 8 + 64 i
  const int a_cc = tid & 7;
  int64_t a_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min((tid >> 3) + 64 * i, valid_rows - 1);
    const int srow = seg + row0 + r;
    a_row[i] = AMODE == MX_GATHER ? g.sorted_pair[srow] / g.topk : srow;
  }
  // weight rows: thread owns 32 bytes (one half) of tile column tid / 2
  const int w_c = tid >> 1, w_half = tid & 1;
  int w_row;
  if (EPI == MX_SWIGLU) {
    const int cw = w_c >> 7, j = (w_c & 127) >> 5, ll = w_c & 31;
    const int pair = nt * (kBN / 2) + cw * 64 + (j & 1) * 32 + ll;
    w_row = pair < g.I ? pair + (j >= 2 ? g.I : 0) : 0;
  } else {
    w_row = nt * kBN + w_c;
    w_row = w_row < g.N ? w_row : 0;
  }
  const uint8_t *wp = g.Wp + int64_t(e) * g.w_e_bytes + int64_t(w_row) * (g.K >> 1) + w_half * 32;
  // scale rows: threads 0..255 the weight rows, 256..511 the activation rows
  const int s_r = tid & 255;
  const uint8_t *ssrc;
  if (tid < 256) {
    int r;
    if (EPI == MX_SWIGLU) {
      const int cw = s_r >> 7, j = (s_r & 127) >> 5, ll = s_r & 31;
      const int pair = nt * (kBN / 2) + cw * 64 + (j & 1) * 32 + ll;
      r = pair < g.I ? pair + (j >= 2 ? g.I : 0) : 0;
    } else {
      r = nt * kBN + s_r;
      r = r < g.N ? r : 0;
    }
    ssrc = g.Ws + int64_t(e) * g.w_e_blocks + int64_t(r) * (g.K >> 5);
  } else {
    const int rr = min(s_r, valid_rows - 1);
    const int srow = seg + row0 + rr;
    const int64_t arow = AMODE == MX_GATHER ? g.sorted_pair[srow] / g.topk : srow;
    ssrc = g.As + arow * (g.K >> 5);
  }

  u32x4 ra[4], rw[2];
  uint32_t rs;
  auto load = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = *reinterpret_cast<const u32x4 *>(g.A + a_row[i] * g.K + ks * kMxK + a_cc * 16);
#pragma unroll
    for (int d = 0; d < 2; ++d)
      rw[d] = *reinterpret_cast<const u32x4 *>(wp + ks * (kMxK / 2) + d * 16);
    rs = *reinterpret_cast<const uint32_t *>(ssrc + ks * 4);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4 *>(&sA[buf][((tid >> 3) + 64 * i) * kMxA + a_cc * 16]) = ra[i];
#pragma unroll
    for (int d = 0; d < 2; ++d)
      *reinterpret_cast<u32x4 *>(&sW[buf][w_c * kMxW + w_half * 32 + d * 16]) = rw[d];
    if (tid < 256) sWs[buf][s_r] = rs;
    else sAs[buf][s_r] = rs;
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const bool wave_active = wm * 64 < valid_rows;
  const int h = lane >> 5;

  auto compute = [&](int cur) {
    if (!wave_active) return;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      i32x8 wf[4], af[2];
      int wsc[4], asc[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = wn * 128 + j * 32 + (lane & 31);
        const u32x4 q = *reinterpret_cast<const u32x4 *>(&sW[cur][n * kMxW + kh * 32 + h * 16]);
        wf[j] = i32x8{int(q[0]), int(q[1]), int(q[2]), int(q[3]), 0, 0, 0, 0};
        wsc[j] = int((sWs[cur][n] >> (8 * (2 * kh + h))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = wm * 64 + i * 32 + (lane & 31);
        const uint8_t *p = &sA[cur][m * kMxA + kh * 64 + h * 16];
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 32);
        af[i] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                      int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
        asc[i] = int((sAs[cur][m] >> (8 * (2 * kh + h))) & 0xFFu);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf[j], af[i], acc[i][j], 4, 0, 0, wsc[j], 0, asc[i]);
      __builtin_amdgcn_s_setprio(0);
    }
  };

  const int nK = g.K / kMxK;
  load(0);
  store(0);
  if (nK > 1) load(1);
  __syncthreads();
  const bool store_first = wave >= 4;
  for (int ks = 0; ks < nK; ++ks) {
    const int cur = ks & 1;
    if (store_first) {
      if (ks + 1 < nK) store(cur ^ 1);
      if (ks + 2 < nK) load(ks + 2);
      compute(cur);
    } else {
      compute(cur);
      if (ks + 1 < nK) store(cur ^ 1);
      if (ks + 2 < nK) load(ks + 2);
    }
    __syncthreads();
  }

  // ---- epilogue: acc[i][j][4q + t] = D[column wn*128 + j*32 + 8q + 4(lane/32) + t]
  //      [row wm*64 + i*32 + lane%32] ----
  const int lrow = wm * 64 + (lane & 31);
  const int lcol = wn * 128 + 4 * (lane >> 5);
  if (EPI == MX_STORE) {
    // through LDS in two halves of 128 rows (the activation stages, bf16, row
    // stride kOut), so that every store is 16 contiguous bytes and a wave
    // writes two 512-byte row segments; the K loop's last barrier has retired
    // every read of the stages
    constexpr int kOut = kBN + 8;
    static_assert(128 * kOut * 2 <= int(sizeof(sA)), "half a tile fits the activation stages");
    uint16_t *otile = reinterpret_cast<uint16_t *>(&sA[0][0]);
    const int cc = (tid & 31) * 8, col = nt * kBN + cc;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if ((wm >> 1) == hf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = (lrow + i * 32) & 127;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x16 &a = acc[i][j];
              *reinterpret_cast<u32x2 *>(otile + r * kOut + lcol + j * 32 + 8 * q) =
                  u32x2{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
            }
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int pass = 0; pass < 128 / 16; ++pass) {
        const int r = pass * 16 + (tid >> 5), row = hf * 128 + r;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(otile + r * kOut + cc);
        if (row < valid_rows && col < g.N)
          *reinterpret_cast<u32x4 *>(g.C + int64_t(seg + row0 + row) * g.ldc + col) = v;
      }
      __syncthreads();
    }
  } else {
    // a = bf16(silu(g) * u) converted to MXFP8 in place: for (i, jj) a lane
    // holds pairs 8 q + 4 (lane / 32) + t of one 32-pair MX block of its row,
    // lane ^ 32 the other sixteen; the block's amax and the stored bytes are
    // exchanged between the two, and each writes 16 of the block's 32 bytes
    const int h2 = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = lrow + i * 32;
      const int64_t grow = seg + row0 + row;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int blk0 = nt * (kBN / 2) + wn * 64 + jj * 32;  // 32-aligned, wave-uniform
        if (blk0 >= g.I) continue;
        float av[4][4];
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float gv = acc[i][jj][4 * q + t], uv = acc[i][jj + 2][4 * q + t];
            const float v = bf16_lo(f32_to_bf16(gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv));
            av[q][t] = v;
            amax = fmaxf(amax, fabsf(v));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int sh = mx8_shared(amax);
        uint32_t wq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)  // bytes of each element pair stored swapped
          wq[q] = e4m3_code(av[q][1], sh) | e4m3_code(av[q][0], sh) << 8 |
                  e4m3_code(av[q][3], sh) << 16 | e4m3_code(av[q][2], sh) << 24;
        // lane h2 = 0 keeps bytes 0..15 (words q = 0, 1 of both lanes),
        // lane h2 = 1 bytes 16..31 (q = 2, 3)
        const uint32_t r0 = __shfl_xor(h2 ? wq[0] : wq[2], 32);
        const uint32_t r1 = __shfl_xor(h2 ? wq[1] : wq[3], 32);
        const u32x4 outw = h2 ? u32x4{r0, wq[2], r1, wq[3]} : u32x4{wq[0], r0, wq[1], r1};
        if (row < valid_rows) {
          *reinterpret_cast<u32x4 *>(g.Cq + grow * g.I + blk0 + 16 * h2) = outw;
          if (h2 == 0) g.Cs[grow * (g.I >> 5) + (blk0 >> 5)] = uint8_t(sh + 127);
        }
      }
    }
  }
}

hipError_t launch_mx8_rows(const uint16_t *x, int64_t rows, int64_t K, uint8_t *codes,
                           uint8_t *scales, hipStream_t s) {
  const int64_t nblocks = rows * (K / kMxBlock);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx8_rows_kernel, dim3(uint32_t((nblocks + 255) / 256)), dim3(256), 0, s, x,
                     nblocks, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(bool gate_up, const MxGemmArgs &a, hipStream_t s,
                          const e4b_kernel_events *ev) {
  if (a.grid == 0) return hipSuccess;
  const dim3 grid{(a.grid + 7) / 8 * 8};
  if (gate_up)
    return launch_k(ev, E4B_K_GATE_UP_FWD, mx_gemm_kernel<MX_GATHER, MX_SWIGLU>, grid, dim3(512), s, a);
  return launch_k(ev, E4B_K_DOWN_FWD, mx_gemm_kernel<MX_DIRECT, MX_STORE>, grid, dim3(512), s, a);
}

}  // namespace e4b

using namespace e4b;

extern "C" e4b_status e4b_mx8_rows(const void *x_bf16, int64_t rows, int64_t K, uint8_t *codes,
                                   uint8_t *scales, hipStream_t stream) {
  if (!x_bf16 || !codes || !scales) return E4B_ERR_NULL;
  if (rows < 0 || K <= 0 || K % kMxBlock != 0 || rows * K > (int64_t(1) << 40)) return E4B_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales)) return E4B_ERR_ALIGN;
  return launch_mx8_rows(static_cast<const uint16_t *>(x_bf16), rows, K, codes, scales,
                         stream) == hipSuccess
             ? E4B_OK
             : E4B_ERR_HIP;
}
