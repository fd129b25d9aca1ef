// encode_bulk.hip -- prefill-side HashEncode of long row runs on the matrix cores.
//
// HATA paper notes, section "Overall framework" (prefill: attention as usual
// while the keys are encoded into binary hash codes and cached) and section
// "Key design: Decode-stage algorithm" (HashEncode = matrix multiply + Sign +
// BitPack).  For N cached keys this is a dense [N x 128] x [128 x 128]
// product per KV head, so it runs on v_mfma_f32_32x32x16_bf16.
//
// Precision: the keys are bf16 already; W_H (fp32) is split exactly into
// three bf16 terms W1 + W2 + W3 (each residual of a bf16 rounding fits in the
// next term), so every product is exact and the fp32 accumulation inside the
// MFMA is the only rounding -- the same order of error as an fp32 GEMV.  On
// inputs whose projections are exact in fp32 the codes are bit-identical to
// the GEMV path.
//
// Work split: workgroup = 4 waves; wave w owns output columns [32w, 32w+32)
// and keeps its three split fragments of W_H for all 128 input channels in
// registers (8 k-steps x 3 x 8 bf16).  A tile of 128 rows is staged in LDS
// (bf16, padded rows) and shared by the 4 waves; the next tile is loaded into
// registers while the current one is multiplied.  Signs are packed straight
// from the accumulator layout with ballots: for accumulator element i, lanes
// 0-31 hold row 8*(i/4) + (i%4) and lanes 32-63 the row 4 below, at columns
// 32w + lane%32, i.e. 32-bit word w of the code.
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 128;
constexpr int kXsStride = kD + 8;  // bf16 elements per staged row (pad: 272 bytes)

__global__ __launch_bounds__(kNT) void encode_bulk_kernel(
    const uint16_t* __restrict__ x, int64_t x_rows, int H, int Hkv, int n_new,
    const float* __restrict__ W, uint64_t* __restrict__ codes, int64_t cap,
    const int32_t* __restrict__ pos, int pos_off, int tiles_per_wg) {
  __shared__ __align__(16) uint16_t xs[kTileRows * kXsStride];
  __shared__ uint32_t cw[kTileRows * 4];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int Gh = H / Hkv;
  const int bh = blockIdx.y;
  const int b = bh / H, hh = bh - b * H, hk = hh / Gh;
  const int total_tiles = (n_new + kTileRows - 1) / kTileRows;
  const int tile0 = blockIdx.x * tiles_per_wg;
  const int tile1 = min(total_tiles, tile0 + tiles_per_wg);
  if (tile0 >= tile1) return;

  // split fragments of W_H: k = 16*s + 8*(lane/32) + j, n = 32*wv + lane%32
  const float* Wh = W + (int64_t)hk * kD * kR;
  bf16x8 w1[8], w2[8], w3[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = Wh[(16 * s + 8 * (lane >> 5) + j) * kR + 32 * wv + (lane & 31)];
      const __bf16 a1 = (__bf16)v;
      const float r1 = v - (float)a1;
      const __bf16 a2 = (__bf16)r1;
      const float r2 = r1 - (float)a2;
      w1[s][j] = a1;
      w2[s][j] = a2;
      w3[s][j] = (__bf16)r2;
    }
  }

  const int64_t p_b = (pos ? (int64_t)pos[b] : 0) + pos_off;
  const int64_t lim = x_rows < cap ? x_rows : cap;
  const int64_t head = (int64_t)b * H + hh;
  const uint16_t* xh = x + head * x_rows * kD;

  // row tile loader: 128 rows x 16 chunks of 16 bytes, 8 chunks per thread
  auto load_tile = [&](int tile, uint4 (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = t + i * kNT, row = c >> 4, c16 = c & 15;
      const int j = tile * kTileRows + row;
      const int64_t ridx = p_b + j;
      v[i] = make_uint4(0, 0, 0, 0);
      if (j < n_new && ridx >= 0 && ridx < lim)
        v[i] = *reinterpret_cast<const uint4*>(xh + ridx * kD + c16 * 8);
    }
  };
  uint4 nxt[8];
  load_tile(tile0, nxt);
  for (int tile = tile0; tile < tile1; ++tile) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = t + i * kNT, row = c >> 4, c16 = c & 15;
      *reinterpret_cast<uint4*>(xs + row * kXsStride + c16 * 8) = nxt[i];
    }
    __syncthreads();
    if (tile + 1 < tile1) load_tile(tile + 1, nxt);
    f32x16 acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][i] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(
            xs + (rt * 32 + (lane & 31)) * kXsStride + 16 * s + 8 * (lane >> 5));
        acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, w1[s], acc[rt], 0, 0, 0);
        acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, w2[s], acc[rt], 0, 0, 0);
        acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, w3[s], acc[rt], 0, 0, 0);
      }
    }
    // sign + pack: 32-bit word wv of rows 8*(i/4) + (i%4) (+4 for lanes 32..63)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint64_t m = __ballot(acc[rt][i] >= 0.0f);
        if (lane == 0) {
          const int row = rt * 32 + 8 * (i >> 2) + (i & 3);
          cw[row * 4 + wv] = (uint32_t)m;
          cw[(row + 4) * 4 + wv] = (uint32_t)(m >> 32);
        }
      }
    }
    __syncthreads();
    if (t < kTileRows) {
      const int j = tile * kTileRows + t;
      const int64_t ridx = p_b + j;
      if (j < n_new && ridx >= 0 && ridx < lim) {
        const uint4 v = make_uint4(cw[t * 4], cw[t * 4 + 1], cw[t * 4 + 2], cw[t * 4 + 3]);
        *reinterpret_cast<uint4*>(codes + (head * cap + ridx) * 2) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_encode_bulk(const uint16_t* x, int64_t x_rows, int B, int H, int Hkv, int n_new,
                              const float* W, uint64_t* codes, int64_t cap, const int32_t* pos,
                              int pos_off, hipStream_t s) {
  const int heads = B * H;
  const int total_tiles = (n_new + kTileRows - 1) / kTileRows;
  // about two workgroups per CU over the launch (256 CUs), W_H fragments
  // loaded once per workgroup
  int wg_per_head = (512 + heads - 1) / heads;
  if (wg_per_head > total_tiles) wg_per_head = total_tiles;
  if (wg_per_head < 1) wg_per_head = 1;
  const int tiles_per_wg = (total_tiles + wg_per_head - 1) / wg_per_head;
  wg_per_head = (total_tiles + tiles_per_wg - 1) / tiles_per_wg;
  hipLaunchKernelGGL(encode_bulk_kernel, dim3(wg_per_head, heads), dim3(kNT), 0, s, x, x_rows, H,
                     Hkv, n_new, W, codes, cap, pos, pos_off, tiles_per_wg);
  return hipGetLastError();
}

}  // namespace hata
