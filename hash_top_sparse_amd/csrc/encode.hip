// encode.hip -- HashEncode (projection by W_H, sign, bit-pack) with cache append.
//
// HATA paper notes, section "Key design: Decode-stage algorithm" (HashEncode =
// matrix multiply + Sign + BitPack, then append the key code to the code
// cache) and section "Hardware-efficient optimisation" (projection, sign,
// bit-pack and cache update fused in one kernel).  bit c = (p_c >= 0.0f),
// word c/64, bit c%64.
//
// GEMV form for a few rows per (sequence, KV head): a 256-thread workgroup
// holds the KV head's W_H in registers (16 rows of r/32 columns per thread)
// and packs each 64-column word of a code with one wave64 ballot
// (project_pack); the fused decode step uses the same routine, so both
// produce identical codes.  Code widths r = 32, 64, 128, 256.
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

constexpr int kRowsPerBatch = 4;

// PAGED: x and codes are page pools addressed through pm (H == Hkv).
template <int R, bool PAGED>
__global__ __launch_bounds__(kNT) void encode_rows_kernel(
    const uint16_t* __restrict__ x, int64_t x_rows, int H, int Hkv, int n_new,
    const float* __restrict__ W, uint32_t* __restrict__ codes, int64_t cap,
    const int32_t* __restrict__ pos, int pos_off, int rows_per_block, PageMap pm) {
  constexpr int W64 = Width<R>::W64, W32 = Width<R>::W32;
  __shared__ __align__(16) float xs[kRowsPerBatch * kD];
  __shared__ __align__(16) float red[4 * kRowsPerBatch * R];
  __shared__ uint64_t cw[kRowsPerBatch * W64];
  const int t = threadIdx.x;
  const int G = H / Hkv;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, hk = bh - b * Hkv;

  const int total = G * n_new;
  const int r_begin = blockIdx.x * rows_per_block;
  const int r_end = min(total, r_begin + rows_per_block);
  if (r_begin >= r_end) return;

  WRegs<R> wr;
  load_w_regs<R>(W + (int64_t)hk * kD * R, wr);

  const int64_t p_b = (pos ? (int64_t)pos[b] : 0) + pos_off;
  const int64_t lim = x_rows < cap ? x_rows : cap;

  for (int r0 = r_begin; r0 < r_end; r0 += kRowsPerBatch) {
    // stage up to 4 rows (64 threads per row, 2 bf16 each)
    {
      const int rr = t >> 6, c2 = t & 63;
      const int r = r0 + rr;
      float lo = 0.f, hi = 0.f;
      if (r < r_end) {
        const int g = r / n_new, j = r - g * n_new;
        const int64_t ridx = p_b + j;
        if (ridx >= 0 && ridx < lim) {
          const int64_t head = (int64_t)b * H + (int64_t)hk * G + g;
          const int64_t xr = PAGED ? pm.row(b, hk, Hkv, ridx) : head * x_rows + ridx;
          const uint32_t two = reinterpret_cast<const uint32_t*>(x + xr * kD)[c2];
          lo = bf16_lo(two);
          hi = bf16_hi(two);
        }
      }
      xs[rr * kD + 2 * c2] = lo;
      xs[rr * kD + 2 * c2 + 1] = hi;
    }
    __syncthreads();
    const int nr = min(kRowsPerBatch, r_end - r0);
    project_pack<kRowsPerBatch, R>(wr, xs, red, cw, nr);
    // 32-bit word t % W32 of row t / W32
    if (t < nr * W32) {
      const int rr = t / W32, wd = t - rr * W32;
      const int r = r0 + rr;
      const int g = r / n_new, j = r - g * n_new;
      const int64_t ridx = p_b + j;
      if (ridx >= 0 && ridx < lim) {
        const int64_t head = (int64_t)b * H + (int64_t)hk * G + g;
        const int64_t cr = PAGED ? pm.row(b, hk, Hkv, ridx) : head * cap + ridx;
        codes[cr * W32 + wd] = code_word32(cw + rr * W64, wd);
      }
    }
  }
}

template <int R>
void launch_encode_r(dim3 grid, const uint16_t* x, int64_t x_rows, int H, int Hkv, int n_new, const float* W,
                     uint32_t* codes, int64_t cap, const int32_t* pos, int pos_off, int rpb, const PageMap* pm,
                     hipStream_t s) {
  if (pm && pm->bt)
    hipLaunchKernelGGL((encode_rows_kernel<R, true>), grid, dim3(kNT), 0, s, x, x_rows, H, Hkv, n_new, W, codes,
                       cap, pos, pos_off, rpb, *pm);
  else
    hipLaunchKernelGGL((encode_rows_kernel<R, false>), grid, dim3(kNT), 0, s, x, x_rows, H, Hkv, n_new, W, codes,
                       cap, pos, pos_off, rpb, PageMap());
}

}  // namespace

hipError_t launch_encode_rows(const uint16_t* x, int64_t x_rows, int B, int H, int Hkv, int n_new,
                              const float* W, uint32_t* codes, int64_t cap, const int32_t* pos,
                              int pos_off, hipStream_t s, int r, const PageMap* pm) {
  if (pm && pm->bt && H != Hkv) return hipErrorInvalidValue;
  const int G = H / Hkv;
  const int64_t total = (int64_t)G * n_new;
  // enough blocks to cover the chip for long row runs, few rows per block otherwise
  int64_t rpb = (total + 31) / 32;
  if (rpb < 16) rpb = 16;
  rpb = (rpb + kRowsPerBatch - 1) / kRowsPerBatch * kRowsPerBatch;
  const int64_t nbx = (total + rpb - 1) / rpb;
  dim3 grid((unsigned)nbx, (unsigned)(B * Hkv));
  switch (r) {
    case 32: launch_encode_r<32>(grid, x, x_rows, H, Hkv, n_new, W, codes, cap, pos, pos_off, (int)rpb, pm, s); break;
    case 64: launch_encode_r<64>(grid, x, x_rows, H, Hkv, n_new, W, codes, cap, pos, pos_off, (int)rpb, pm, s); break;
    case 256: launch_encode_r<256>(grid, x, x_rows, H, Hkv, n_new, W, codes, cap, pos, pos_off, (int)rpb, pm, s); break;
    default: launch_encode_r<128>(grid, x, x_rows, H, Hkv, n_new, W, codes, cap, pos, pos_off, (int)rpb, pm, s); break;
  }
  return hipGetLastError();
}

__global__ void fill_zero_kernel(unsigned char* p, size_t bytes) {
  const size_t words = bytes / 4;
  uint32_t* w = reinterpret_cast<uint32_t*>(p);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t i = i0; i < words; i += stride) w[i] = 0u;
  for (size_t i = words * 4 + i0; i < bytes; i += stride) p[i] = 0;
}

// Zero `bytes` bytes at p (4-byte aligned) with a kernel, so the reset can be
// captured in a HIP graph.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  size_t blocks = (bytes / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<unsigned char*>(p), bytes);
  return hipGetLastError();
}

__global__ void set_word_kernel(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0) p[0] = v;
}

// Write one 32-bit word of device memory with a kernel (graph-capturable).
hipError_t launch_set_word(uint32_t* p, uint32_t v, hipStream_t s) {
  hipLaunchKernelGGL(set_word_kernel, dim3(1), dim3(64), 0, s, p, v);
  return hipGetLastError();
}

}  // namespace hata
