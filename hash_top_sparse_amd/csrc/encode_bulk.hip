// encode_bulk.hip -- prefill-side HashEncode of long row runs on the matrix cores.
//
// HATA paper notes, section "Overall framework" (prefill: attention as usual
// while the keys are encoded into binary hash codes and cached) and section
// "Key design: Decode-stage algorithm" (HashEncode = matrix multiply + Sign +
// BitPack).  For N cached keys this is a dense [N x 128] x [128 x 128]
// product per KV head, so it runs on v_mfma_f32_32x32x16_bf16.
//
// Precision: the keys are bf16 already; W_H (fp32) is split into two bf16
// terms W1 = bf16(W) and W2 = bf16(W - W1) (both differences exact in fp32).
// Each rounding keeps 8 significant bits, so the residual W - W1 - W2 is at
// most 2^-16 |W| per weight and the projection differs from the exact one by
// at most 2^-16 sum_i |x_i W_i| plus the fp32 accumulation inside the MFMA:
// the worst case of a 128-term fp32 GEMV's own rounding is about 2^-17 of the
// same sum.  A weight with at most 16 significant bits (W_H in {-1, 0, 1},
// multiples of a power of two, ...) is represented exactly, and on inputs
// whose projections are then exact in fp32 the codes are bit-identical to
// the GEMV path.
//
// Work split: workgroup = 4 waves; wave w owns bits [32w, 32w+32) of the
// code and keeps its two split fragments of W_H for all 128 input channels in
// registers (8 k-steps x 2 x 8 bf16).  The product is formed transposed,
// D[bit][row] = W_H^T x^T, so that a lane's accumulators all belong to one
// row (lane % 32) and 16 of the wave's 32 bits (the other 16 in lane ^ 32):
// each lane packs its signs into a word, one lane exchange completes it.
// Tiles of 128 rows are staged in LDS one at a time while the next two are
// in flight in registers; the code words of the workgroup's tiles (at most
// 16) collect in LDS and are stored at the end, so no store sits between the
// loads (a store in flight would make the compiler wait for every load).
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 128;
constexpr int kXsStride = kD + 8;  // bf16 elements per staged row (pad: 272 bytes)
constexpr int kMaxTilesPerWg = 16; // code words of every tile of a workgroup stay in LDS

// TILES: tiles per workgroup (even, at most kMaxTilesPerWg), a compile-time
// count so that the tile loop unrolls into straight-line code
template <int TILES>
__global__ __launch_bounds__(kNT, 2) void encode_bulk_kernel(
    const uint16_t* __restrict__ x, int64_t x_rows, int H, int Hkv, int n_new,
    const float* __restrict__ W, uint32_t* __restrict__ codes, int64_t cap,
    const int32_t* __restrict__ pos, int pos_off) {
  static_assert(TILES % 2 == 0 && TILES <= kMaxTilesPerWg, "tiles per workgroup");
  constexpr int tiles_per_wg = TILES;
  __shared__ __align__(16) uint16_t xs[kTileRows * kXsStride];
  __shared__ __align__(16) uint32_t cw[kMaxTilesPerWg * kTileRows * 4];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int Gh = H / Hkv;
  const int bh = blockIdx.y;
  const int b = bh / H, hh = bh - b * H, hk = hh / Gh;
  const int total_tiles = (n_new + kTileRows - 1) / kTileRows;
  const int tile0 = blockIdx.x * tiles_per_wg;
  if (tile0 >= total_tiles) return;

  // split fragments of W_H^T: bit 32*wv + lane%32, k = 16*s + 8*(lane/32) + j
  const float* Wh = W + (int64_t)hk * kD * kR;
  bf16x8 w1[8], w2[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = Wh[(16 * s + 8 * (lane >> 5) + j) * kR + 32 * wv + (lane & 31)];
      const __bf16 a1 = (__bf16)v;
      w1[s][j] = a1;
      w2[s][j] = (__bf16)(v - (float)a1);
    }
  }

  const int64_t p_b = (pos ? (int64_t)pos[b] : 0) + pos_off;
  const int64_t lim = x_rows < cap ? x_rows : cap;
  const int64_t head = (int64_t)b * H + hh;
  // rows [r_lo, r_hi) of this head are encoded (row p_b + j for j < n_new,
  // inside both the input and the cache); buffer resources over exactly
  // these rows make every load and store branch-free: a row outside reads
  // as zeros and its store is dropped, so the compiler can count the loads
  // in flight and wait for one tile without draining the next
  const int64_t r_lo = p_b > 0 ? p_b : 0;
  const int64_t r_hi = lim < p_b + n_new ? lim : p_b + n_new;
  if (r_hi <= r_lo) return;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (head * x_rows + r_lo) * kD), 0, (int)((r_hi - r_lo) * kD * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      codes + (head * cap + r_lo) * 4, 0, (int)((r_hi - r_lo) * 16), 0x00020000);

  // row tile loader: 128 rows x 16 chunks of 16 bytes, 8 chunks per thread
  // (rows before r_lo give negative offsets, i.e. out of range as well)
  auto load_tile = [&](int tile, uint4 (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = t + i * kNT, row = c >> 4, c16 = c & 15;
      const int64_t rel = p_b + (int64_t)tile * kTileRows + row - r_lo;
      const u32x4 ld = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(rel * (kD * 2) + c16 * 16), 0, 0);
      v[i] = make_uint4(ld.x, ld.y, ld.z, ld.w);
    }
  };
  // One tile: stage the registers `buf` (this tile) in LDS, refill `buf`
  // with tile + 2 (two tiles in flight while one is multiplied; not past the
  // workgroup's last tile), multiply, and keep the tile's code words in LDS
  // slot j.
  auto step = [&](int tile, uint4 (&buf)[8], int j, bool refill) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = t + i * kNT, row = c >> 4, c16 = c & 15;
      *reinterpret_cast<uint4*>(xs + row * kXsStride + c16 * 8) = buf[i];
    }
    __syncthreads();  // tile staged
    if (refill) load_tile(tile + 2, buf);
    f32x16 acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][i] = 0.f;
    // sign + pack of row block rt: accumulator i of lane l is bit
    // 8*(i/4) + 4*(l/32) + i%4 of word wv of row rt*32 + l%32.  The 16 sign
    // bits are shifted into one word (one alignbit each), spread to their
    // nibbles and inverted: a code bit is 1 where the sign bit is clear,
    // which is p >= 0 for every p the accumulation can produce (it starts at
    // +0, and an exact zero sum of fp32 terms rounds to +0, never -0).
    auto pack = [&](int rt) {
      uint32_t neg = 0;
#pragma unroll
      for (int i = 15; i >= 0; --i) neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(acc[rt][i]), 31);
      neg = ((neg & 0xF000u) << 12) | ((neg & 0x0F00u) << 8) | ((neg & 0x00F0u) << 4) | (neg & 0x000Fu);
      uint32_t part = (~neg & 0x0F0F0F0Fu) << (4 * (lane >> 5));
      part |= __shfl_xor(part, 32);
      if (lane < 32) cw[(j * kTileRows + rt * 32 + lane) * 4 + wv] = part;
    };
    // Two halves of two row blocks each: the first half's products, then the
    // second half's with the first half's packing placed among them (vector
    // work that the matrix core's latency hides), then the second half's
    // packing.  Fragments are read one k-step ahead; within a step W1 runs
    // over the half's two accumulators, then W2.
    const uint16_t* xrow = xs + (lane & 31) * kXsStride + 8 * (lane >> 5);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 xf[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        xf[0][q] = *reinterpret_cast<const bf16x8*>(xrow + (2 * hf + q) * 32 * kXsStride);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s + 1 < 8) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
            xf[(s + 1) & 1][q] =
                *reinterpret_cast<const bf16x8*>(xrow + (2 * hf + q) * 32 * kXsStride + 16 * (s + 1));
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
          acc[2 * hf + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1[s], xf[s & 1][q], acc[2 * hf + q], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          acc[2 * hf + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2[s], xf[s & 1][q], acc[2 * hf + q], 0, 0, 0);
        if (hf == 1 && s == 2) pack(0);
        if (hf == 1 && s == 5) pack(1);
      }
    }
    __syncthreads();  // every wave done reading the tile
    pack(2);
    pack(3);
  };
  // Every workgroup runs all TILES tiles: tiles past the rows read zeros and
  // their stores are dropped.  The loop unrolls completely (refill is known
  // at compile time) and issues no store, so the compiler counts the loads in
  // flight exactly and waits for one tile while the next stays in flight.
  uint4 na[8], nb[8];
  load_tile(tile0, na);
  load_tile(tile0 + 1, nb);
#pragma unroll
  for (int j = 0; j < TILES; j += 2) {
    step(tile0 + j, na, j, j + 2 < TILES);
    step(tile0 + j + 1, nb, j + 1, j + 3 < TILES);
  }
  // the code rows: 16 bytes each, tiles_per_wg * 128 of them (the last
  // tile's words come from every wave's pack, hence the barrier)
  __syncthreads();
  for (int e = t; e < tiles_per_wg * kTileRows; e += kNT) {
    const int64_t rel = p_b + (int64_t)tile0 * kTileRows + e - r_lo;
    const u32x4 v = *reinterpret_cast<const u32x4*>(cw + e * 4);
    __builtin_amdgcn_raw_buffer_store_b128(v, cr, (int)(rel * 16), 0, 0);
  }
}

}  // namespace

hipError_t launch_encode_bulk(const uint16_t* x, int64_t x_rows, int B, int H, int Hkv, int n_new,
                              const float* W, uint32_t* codes, int64_t cap, const int32_t* pos,
                              int pos_off, hipStream_t s) {
  // the kernel's buffer resources span at most kMaxRows rows (1 GiB of keys);
  // longer runs are encoded in pieces
  constexpr int kMaxRows = 1 << 22;
  if (n_new > kMaxRows) {
    for (int off = 0; off < n_new; off += kMaxRows) {
      const int m = n_new - off < kMaxRows ? n_new - off : kMaxRows;
      hipError_t e = launch_encode_bulk(x, x_rows, B, H, Hkv, m, W, codes, cap, pos, pos_off + off, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int heads = B * H;
  const int total_tiles = (n_new + kTileRows - 1) / kTileRows;
  // 16 tiles (2048 rows) per workgroup on long runs, 4 on short ones (the
  // last workgroup of a head multiplies zero rows past the run)
  if (total_tiles >= 64) {
    const int wg_per_head = (total_tiles + 15) / 16;
    hipLaunchKernelGGL(encode_bulk_kernel<16>, dim3(wg_per_head, heads), dim3(kNT), 0, s, x, x_rows, H,
                       Hkv, n_new, W, codes, cap, pos, pos_off);
  } else {
    const int wg_per_head = (total_tiles + 3) / 4;
    hipLaunchKernelGGL(encode_bulk_kernel<4>, dim3(wg_per_head, heads), dim3(kNT), 0, s, x, x_rows, H,
                       Hkv, n_new, W, codes, cap, pos, pos_off);
  }
  return hipGetLastError();
}

}  // namespace hata
