// quant.hip -- blockwise absmax 4-bit and 8-bit quantize / dequantize of a
// fused stack, and the bf16 passthrough lane (round to nearest even / widen).
//
// experts4bit-qlora 0.1.0 sdist, _vendor/experts.py: Experts4bit quantizes
// each expert of an [E, out, in] stack on its own with blocksize 64 and
// dequantizes one expert as code value times block absmax. Blocks are 64
// consecutive row-major elements, so the flat index of an element determines
// its block across the whole contiguous [E, out*in/64] absmax array.
#include "codebook8.h"
#include "device.h"
#include "plan.h"

namespace e4b {

// One wavefront per 64-element block, one element per lane.
// absmax = max |w| (exact); the code is decided with fp64 products
// absmax * midpoint, which are exact for fp32 operands, so the decision is the
// true nearest entry (ties: NF4 lower code, FP4 smaller magnitude). This step
// runs once per layer, off the forward/backward path.
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ w,
                                                       int64_t nblocks, int cb,
                                                       uint8_t *__restrict__ packed,
                                                       float *__restrict__ absmax) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;  // whole wave exits together
  const float v = w[blk * 64 + lane];
  float m = fabsf(v);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const double amax = double(m);
  const double x = double(v);
  int q = 0;
  if (cb == E4B_CB_NF4) {
    if (m == 0.0f) {
      q = 7;
    } else {
#pragma unroll
      for (int i = 0; i < 15; ++i) {
        const double mid = (double(codebook_value(0, i)) + double(codebook_value(0, i + 1))) * 0.5;
        q += x > amax * mid ? 1 : 0;
      }
    }
  } else {
    const double ax = fabs(x);
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      const double mid = (double(codebook_value(1, i)) + double(codebook_value(1, i + 1))) * 0.5;
      q += ax > amax * mid ? 1 : 0;
    }
    q += signbit(v) ? 8 : 0;
  }
  const int q_next = __shfl_down(q, 1);
  if ((lane & 1) == 0) packed[blk * 32 + (lane >> 1)] = uint8_t((q << 4) | q_next);
  if (lane == 0) absmax[blk] = m;
}

// MXFP4 conversion (OCP MX v1.0, the reading of the 0.31.1 project page's
// MXFP4 experts): one thread per 32-element block. The shared exponent is
// floor(log2(amax)) - 2 from amax's exponent field (frexpf, exact), clamped
// to [-127, 127]; w * 2^-shared is exact wherever it matters (a product that
// underflows to a subnormal is below 0.25 and rounds to zero either way); the
// E2M1 index is counted against the exact midpoints, with the ties whose lower
// neighbour has an odd mantissa (0.75, 1.75, 3.5) moved up to the even one.
__global__ __launch_bounds__(256) void quantize_mx_kernel(const float *__restrict__ w,
                                                          int64_t nblocks,
                                                          uint8_t *__restrict__ packed,
                                                          uint8_t *__restrict__ scales) {
  const int64_t blk = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(w + blk * kMxBlock);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 q = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * i + j] = q[j];
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int ex = 0;
  frexpf(amax, &ex);  // amax = m * 2^ex, 0.5 <= m < 1
  const int sh = amax == 0.0f ? -127 : min(127, max(-127, ex - 1 - 2));
  uint32_t q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float a = fabsf(ldexpf(v[i], -sh));
    uint32_t m = (a > 0.25f) + (a > 0.75f) + (a > 1.25f) + (a > 1.75f) + (a > 2.5f) +
                 (a > 3.5f) + (a > 5.0f);
    m += (a == 0.75f) | (a == 1.75f) | (a == 3.5f);
    q[i] = m | (signbit(v[i]) ? 8u : 0u);
  }
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= ((q[8 * d + 2 * b] << 4) | q[8 * d + 2 * b + 1]) << (8 * b);
    o[d] = word;
  }
  reinterpret_cast<u32x4 *>(packed)[blk] = o;
  scales[blk] = uint8_t(sh + 127);
}

// One thread per 8 consecutive elements (4 packed bytes). MXFP4 (scales !=
// nullptr): the block scale is the E8M0 byte of the 32-element block.
template <bool BF16>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint32_t *__restrict__ packed,
                                                         const float *__restrict__ absmax,
                                                         const uint8_t *__restrict__ scales,
                                                         int64_t ngroups, int cb,
                                                         void *__restrict__ out) {
  __shared__ float code[16];
  if (threadIdx.x < 16) code[threadIdx.x] = codebook_value(cb, threadIdx.x);
  __syncthreads();
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const uint32_t d = packed[g];
  // 8 groups of 8 elements per 64-block; 4 per 32-element MX block
  const float a = scales ? e8m0_value(scales[g >> 2]) : absmax[g >> 3];
  float v[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[2 * b] = __fmul_rn(code[(d >> (8 * b + 4)) & 15u], a);
    v[2 * b + 1] = __fmul_rn(code[(d >> (8 * b)) & 15u], a);
  }
  if (BF16) {
    u32x4 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
    reinterpret_cast<u32x4 *>(out)[g] = o;
  } else {
    f32x4 *o = reinterpret_cast<f32x4 *>(out) + 2 * g;
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// 8-bit lanes (INT8, FP8): one wavefront per 64-element block, one element
// per lane. The index of |w| / absmax among the 128 ascending magnitudes is
// the number of midpoints m below it, counted by a binary search on the
// exact fp64 products absmax * m (the midpoints of adjacent fp32 magnitudes
// need at most 28 bits), so ties go to the smaller magnitude; the sign bit is
// w's. One code byte per element.
__global__ __launch_bounds__(256) void quantize8_kernel(const float *__restrict__ w, int64_t nblocks,
                                                        int lane8, uint8_t *__restrict__ codes,
                                                        float *__restrict__ absmax) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;  // whole wave exits together
  const float v = w[blk * 64 + lane];
  float m = fabsf(v);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const double amax = double(m), a = fabs(double(v));
  const float *mag = kMag8[lane8].v;
  int lo = 0, hi = 127;  // the count of midpoints below a lies in [lo, hi]
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    const int mid = (lo + hi) >> 1;  // midpoint between magnitudes mid and mid + 1
    const double mp = (double(mag[mid]) + double(mag[mid + 1])) * 0.5;
    if (a > amax * mp) lo = mid + 1;
    else hi = mid;
  }
  codes[blk * 64 + lane] = uint8_t(lo | (signbit(v) ? 0x80 : 0));
  if (lane == 0) absmax[blk] = m;
}

// 8-bit lanes: one thread per 8 consecutive elements (8 code bytes);
// fl32(value(code) * absmax), or its bf16 rounding.
template <bool BF16>
__global__ __launch_bounds__(256) void dequantize8_kernel(const u32x2 *__restrict__ codes,
                                                          const float *__restrict__ absmax,
                                                          int64_t ngroups, int lane8,
                                                          void *__restrict__ out) {
  __shared__ float val[256];
  {
    const float mg = kMag8[lane8].v[threadIdx.x & 127];
    val[threadIdx.x] = threadIdx.x < 128 ? mg : -mg;
  }
  __syncthreads();
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const u32x2 c = codes[g];
  const float a = absmax[g >> 3];
  float v[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) v[b] = __fmul_rn(val[(c[b >> 2] >> (8 * (b & 3))) & 255u], a);
  if (BF16) {
    u32x4 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
    reinterpret_cast<u32x4 *>(out)[g] = o;
  } else {
    f32x4 *o = reinterpret_cast<f32x4 *>(out) + 2 * g;
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

hipError_t launch_dequantize8(const e4b_stack &st, bool bf16, void *out, hipStream_t s) {
  const int64_t ngroups = st.E * st.out * st.in / 8;
  const dim3 grid(uint32_t((ngroups + 255) / 256));
  const u32x2 *c = reinterpret_cast<const u32x2 *>(st.packed);
  const int lane8 = int(st.codebook) - E4B_CB_INT8;
  if (bf16)
    hipLaunchKernelGGL(dequantize8_kernel<true>, grid, dim3(256), 0, s, c, st.absmax, ngroups, lane8, out);
  else
    hipLaunchKernelGGL(dequantize8_kernel<false>, grid, dim3(256), 0, s, c, st.absmax, ngroups, lane8, out);
  return hipGetLastError();
}

// BF16 passthrough lane: one thread per 8 elements, round to nearest even.
__global__ __launch_bounds__(256) void quantize_bf16_kernel(const float *__restrict__ w,
                                                            int64_t ngroups,
                                                            uint16_t *__restrict__ out) {
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(w) + 2 * g;
  const f32x4 a = src[0], b = src[1];
  reinterpret_cast<u32x4 *>(out)[g] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                            pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
}

// BF16 stack -> fp32 (exact) or bf16 (copy); one thread per 8 elements.
template <bool BF16>
__global__ __launch_bounds__(256) void dequantize_bf16_kernel(const u32x4 *__restrict__ in,
                                                              int64_t ngroups,
                                                              void *__restrict__ out) {
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const u32x4 q = in[g];
  if (BF16) {
    reinterpret_cast<u32x4 *>(out)[g] = q;
  } else {
    f32x4 *o = reinterpret_cast<f32x4 *>(out) + 2 * g;
    o[0] = f32x4{bf16_lo(q[0]), bf16_hi(q[0]), bf16_lo(q[1]), bf16_hi(q[1])};
    o[1] = f32x4{bf16_lo(q[2]), bf16_hi(q[2]), bf16_lo(q[3]), bf16_hi(q[3])};
  }
}

}  // namespace e4b

using namespace e4b;

extern "C" e4b_status e4b_quantize_nf4(const float *w, int64_t E, int64_t out, int64_t in,
                                       int32_t blocksize, int32_t codebook, uint8_t *packed,
                                       float *absmax, hipStream_t stream) {
  e4b_status s = check_quantize(w, E, out, in, blocksize, codebook, packed, absmax);
  if (s != E4B_OK) return s;
  if (codebook == E4B_CB_BF16) {
    const int64_t ngroups = E * out * in / 8;
    hipLaunchKernelGGL(quantize_bf16_kernel, dim3(uint32_t((ngroups + 255) / 256)), dim3(256), 0,
                       stream, w, ngroups, reinterpret_cast<uint16_t *>(packed));
    return hipGetLastError() == hipSuccess ? E4B_OK : E4B_ERR_HIP;
  }
  const int64_t nblocks = E * out * in / kBlock;
  const int64_t grid = (nblocks + 3) / 4;
  if (codebook == E4B_CB_INT8 || codebook == E4B_CB_FP8)
    hipLaunchKernelGGL(quantize8_kernel, dim3(uint32_t(grid)), dim3(256), 0, stream, w, nblocks,
                       int(codebook) - E4B_CB_INT8, packed, absmax);
  else
    hipLaunchKernelGGL(quantize_kernel, dim3(uint32_t(grid)), dim3(256), 0, stream, w, nblocks,
                       int(codebook), packed, absmax);
  return hipGetLastError() == hipSuccess ? E4B_OK : E4B_ERR_HIP;
}

extern "C" e4b_status e4b_quantize_mxfp4(const float *w, int64_t E, int64_t out, int64_t in,
                                         uint8_t *packed, uint8_t *scales, hipStream_t stream) {
  e4b_status s = check_quantize_mx(w, E, out, in, packed, scales);
  if (s != E4B_OK) return s;
  const int64_t nblocks = E * out * in / kMxBlock;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3(uint32_t((nblocks + 255) / 256)), dim3(256), 0,
                     stream, w, nblocks, packed, scales);
  return hipGetLastError() == hipSuccess ? E4B_OK : E4B_ERR_HIP;
}

extern "C" e4b_status e4b_dequantize_nf4(const e4b_stack *st, int32_t dtype, void *w_out,
                                         hipStream_t stream) {
  e4b_status s = check_stack(st);
  if (s != E4B_OK) return s;
  if (!w_out) return E4B_ERR_NULL;
  if (dtype != E4B_F32 && dtype != E4B_BF16) return E4B_ERR_DTYPE;
  if (!aligned16(w_out)) return E4B_ERR_ALIGN;
  const int64_t ngroups = st->E * st->out * st->in / 8;
  const int64_t grid = (ngroups + 255) / 256;
  if (st->codebook == E4B_CB_BF16) {
    const u32x4 *in = reinterpret_cast<const u32x4 *>(st->packed);
    if (dtype == E4B_BF16)
      hipLaunchKernelGGL(dequantize_bf16_kernel<true>, dim3(uint32_t(grid)), dim3(256), 0, stream,
                         in, ngroups, w_out);
    else
      hipLaunchKernelGGL(dequantize_bf16_kernel<false>, dim3(uint32_t(grid)), dim3(256), 0, stream,
                         in, ngroups, w_out);
    return hipGetLastError() == hipSuccess ? E4B_OK : E4B_ERR_HIP;
  }
  if (st->codebook == E4B_CB_INT8 || st->codebook == E4B_CB_FP8)
    return launch_dequantize8(*st, dtype == E4B_BF16, w_out, stream) == hipSuccess ? E4B_OK : E4B_ERR_HIP;
  const uint32_t *pk = reinterpret_cast<const uint32_t *>(st->packed);
  const bool mx = st->codebook == E4B_CB_MXFP4;
  const float *am = mx ? nullptr : st->absmax;
  const uint8_t *sc = mx ? st->scales : nullptr;
  if (dtype == E4B_BF16)
    hipLaunchKernelGGL(dequantize_kernel<true>, dim3(uint32_t(grid)), dim3(256), 0, stream, pk,
                       am, sc, ngroups, int(st->codebook), w_out);
  else
    hipLaunchKernelGGL(dequantize_kernel<false>, dim3(uint32_t(grid)), dim3(256), 0, stream, pk,
                       am, sc, ngroups, int(st->codebook), w_out);
  return hipGetLastError() == hipSuccess ? E4B_OK : E4B_ERR_HIP;
}

extern "C" e4b_status e4b_stack_copy_async(const e4b_stack *dst, const e4b_stack *src,
                                           hipStream_t stream) {
  e4b_status s = check_stack(dst);
  if (s != E4B_OK) return s;
  s = check_stack(src);
  if (s != E4B_OK) return s;
  if (dst->E != src->E || dst->out != src->out || dst->in != src->in ||
      dst->codebook != src->codebook)
    return E4B_ERR_SHAPE;
  const int64_t n = dst->E * dst->out * dst->in;
  const bool bf16 = dst->codebook == E4B_CB_BF16;
  const bool w8 = dst->codebook == E4B_CB_INT8 || dst->codebook == E4B_CB_FP8;
  if (hipMemcpyAsync(const_cast<uint8_t *>(dst->packed), src->packed,
                     size_t(bf16 ? n * 2 : w8 ? n : n / 2), hipMemcpyDefault, stream) != hipSuccess)
    return E4B_ERR_HIP;
  if (dst->codebook == E4B_CB_MXFP4) {
    if (hipMemcpyAsync(const_cast<uint8_t *>(dst->scales), src->scales, size_t(n / kMxBlock),
                       hipMemcpyDefault, stream) != hipSuccess)
      return E4B_ERR_HIP;
  } else if (!bf16 && hipMemcpyAsync(const_cast<float *>(dst->absmax), src->absmax,
                                     size_t(n / kBlock) * sizeof(float), hipMemcpyDefault,
                                     stream) != hipSuccess) {
    return E4B_ERR_HIP;
  }
  return E4B_OK;
}
