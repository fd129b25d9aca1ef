// hata_launch.hpp -- host-side launchers of the HATA kernels (internal to libhata.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hata {

// A paged cache (PagedAttention-style block table): row j of (sequence b,
// KV head h) lives in page bt[b * max_pages + j / P] of a pool laid out
// [pages][Hkv][P][row], P = 2^log2P.  Page ids outside [0, num_pages) are
// clamped into it, so the accesses stay inside the pool.
struct PageMap {
  const int32_t* bt = nullptr;
  int max_pages = 0, num_pages = 0, log2P = 0;
  __device__ __forceinline__ int64_t row(int b, int h, int Hkv, int64_t j) const { return at(page(b, j), h, Hkv, j); }
  // the pool page holding row j of sequence b (the id clamped into the pool)
  __device__ __forceinline__ int page(int b, int64_t j) const {
    const int pg = bt[(int64_t)b * max_pages + (int)(j >> log2P)];
    return min(max(pg, 0), num_pages - 1);
  }
  // pool row of row j of a sequence whose page for j is pg
  __device__ __forceinline__ int64_t at(int pg, int h, int Hkv, int64_t j) const {
    return (((int64_t)pg * Hkv + h) << log2P) + (j & ((int64_t(1) << log2P) - 1));
  }
};

// ---------------------------------------------------------------- encode
// x bf16 [B][H][x_rows][128]; rows p_b + j (j < n_new) -> codes [B][H][cap][2].
// Row index of (b, j) is (pos ? pos[b] : 0) + pos_off + j.
hipError_t launch_encode_rows(const uint16_t* x, int64_t x_rows, int B, int H, int Hkv, int n_new,
                              const float* W, uint32_t* codes, int64_t cap, const int32_t* pos,
                              int pos_off, hipStream_t s, int r = 128, const PageMap* pm = nullptr);
// Same contract, matrix-core path for long row runs (prefill).
hipError_t launch_encode_bulk(const uint16_t* x, int64_t x_rows, int B, int H, int Hkv, int n_new,
                              const float* W, uint32_t* codes, int64_t cap, const int32_t* pos,
                              int pos_off, hipStream_t s);
// Row-run length from which hata_encode_append uses the matrix-core path.
constexpr int kBulkMinRows = 512;

// ---------------------------------------------------------------- score / select
hipError_t launch_hamming(const uint32_t* qc, const uint32_t* kc, int B, int Hq, int Hkv,
                          int64_t cap, const int32_t* seq_lens, int64_t max_len, uint16_t* scores,
                          int64_t sstride, hipStream_t s, int r = 128, const PageMap* pm = nullptr,
                          uint32_t* hist = nullptr);
// scratch (optional, topk_scratch_bytes bytes, no initialisation needed):
// with it, sequences longer than 4096 rows are selected by many workgroups
// per unit; the result is the same.  max_len bounds the sequence lengths.
size_t topk_scratch_bytes(int B, int Hkv, int64_t max_len, int max_score);
hipError_t launch_topk(const uint16_t* scores, int64_t sstride, int B, int Hkv, int64_t cap,
                       const int32_t* seq_lens, int k, int max_score, int32_t* idx, hipStream_t s,
                       void* scratch = nullptr, int64_t max_len = 0);
// The same selection when launch_hamming already filled the unit histograms
// (hist = the start of scratch, zeroed before the Hamming launch).
hipError_t launch_topk_after_hamming(const uint16_t* scores, int64_t sstride, int B, int Hkv, int64_t cap,
                                     const int32_t* seq_lens, int k, int max_score, int32_t* idx, hipStream_t s,
                                     void* scratch, int64_t max_len);

// ---------------------------------------------------------------- attention
// Split-K partial attention + combine.  idx == nullptr means dense (rows
// [0, n_b)).  part: workspace of attn_part_floats(...) floats.
size_t attn_part_floats(int B, int Hkv, int G, int64_t max_rows);
hipError_t launch_attention(const uint16_t* q, const uint16_t* K, const uint16_t* V, int B, int Hq,
                            int Hkv, int64_t cap, const int32_t* idx, int k,
                            const int32_t* seq_lens, int64_t max_len, float scale, float* out,
                            float* part, hipStream_t s, const PageMap* pm = nullptr);

// ---------------------------------------------------------------- fused step
struct StepPlan {
  bool fused = false;
  int G = 0, U = 0, Wg = 1, chunk = 0, xcd_map = 0, R = 128;
  size_t lds_bytes = 0;
  // workspace layout (byte offsets)
  size_t off_err = 0, off_flags = 0, off_stamps = 0, off_win = 0, off_full = 0, off_part = 0;
  size_t off_qc = 0, off_scores = 0, off_idx = 0, off_attn = 0, off_topk = 0;
  size_t off_trace = 0;  // phase-trace build only: per-workgroup timestamps at the end
  size_t off_xend = 0;   // end of the exchange area (error words, flags, stamps, windows)
  int full_words = 0;  // 32-bit words per workgroup in the full-histogram area
  size_t total = 0;
};
StepPlan plan_decode_step(int B, int Hq, int Hkv, int64_t max_len, int k, int num_cus, int r = 128);

// hata_decode_step_noalloc: a static device array of this many bytes per
// device serves as the step's workspace; noalloc_scratch gives its address
// on the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(unsigned char** out);
hipError_t launch_decode_step(const StepPlan& p, const uint16_t* q, const uint16_t* K,
                              const uint16_t* V, const float* W, const float* Wk, uint32_t* codes, int B, int Hq,
                              int Hkv, int64_t cap, const int32_t* seq_lens, int k, float scale,
                              float* out, int32_t* idx_out, unsigned char* ws, hipStream_t s);

// The fused step over a paged cache (K, V, codes in page pools, pm): plans
// whose step is fused, any code width, any page size of at least 16 rows,
// while the page-id list still fits in LDS beside the step's own.
bool decode_step_paged_fusable(const StepPlan& p, int page_rows);
hipError_t launch_decode_step_paged(const StepPlan& p, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                    const float* W, uint32_t* codes, const PageMap& pm, int Hq, int Hkv,
                                    const int32_t* seq_lens, int k, float scale, float* out, int32_t* idx_out,
                                    unsigned char* ws, hipStream_t s);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_set_word(uint32_t* p, uint32_t v, hipStream_t s);

// ---------------------------------------------------------------- prefill
// Causal attention over each sequence's prompt (queries [B][Hq][q_rows][128]
// at positions 0..n_b-1, keys/values [B][Hkv][cap][128]) into out fp32
// [B][Hq][q_rows][128], with code rows 0..n_b-1 written to codes
// [B][Hkv][cap][r/32] 32-bit words; n_b = min(seq_lens[b], max_len).
// G = Hq / Hkv in {1, 2, 4, 8}, r in {32, 64, 128, 256}.  pm (optional): K, V
// and codes are page pools addressed through it (cap = max_pages * P).
int prefill_positions_per_block(int G);
hipError_t launch_prefill(const uint16_t* q, const uint16_t* K, const uint16_t* V, const float* W,
                          uint32_t* codes, int B, int Hq, int Hkv, int64_t q_rows, int64_t cap,
                          const int32_t* seq_lens, int max_len, float scale, float* out, int r,
                          hipStream_t s, const PageMap* pm = nullptr);

// training step of the hash weights (train.hip)
constexpr int kMaxLabelKeys = 8192;  // keys a label row may rank (LDS sort)
struct TrainPlan {
  size_t hq = 0, hk = 0, shk = 0, sthq = 0, cm = 0, mtc = 0, rs = 0, cs = 0, dzq = 0, dzk = 0, gram = 0,
         dw = 0, wa = 0, partq = 0, partk = 0, fac = 0, part = 0, total = 0;
};
TrainPlan plan_train(int J, int n, int r);
int train_gemm_splits(int M, int N, int K);
size_t label_lds_bytes(int n, int pos_permille);
hipError_t launch_hash_labels(const uint16_t* q, const uint16_t* k, const int32_t* q_pos, int J, int n,
                              int pos_permille, float s_max, float s_min, float* S, hipStream_t s);
hipError_t launch_hash_train_step(const TrainPlan& p, const uint16_t* q, const uint16_t* k, const int32_t* q_pos,
                                  const float* S, int J, int n, int r, float sigma, float eps, float eta,
                                  float lam, float lr, float* W, float* grad, float* loss, unsigned char* ws,
                                  hipStream_t s);

// read-only streaming reduction (measurement of the device's HBM read rate)
int stream_read_blocks();
hipError_t launch_stream_read(const void* src, size_t bytes, uint64_t* sink, int blocks, hipStream_t s);

}  // namespace hata
