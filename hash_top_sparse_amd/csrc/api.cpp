// api.cpp -- the C ABI of libhata.so: argument validation, workspace layout
// and kernel dispatch.  Declarations and the full contract are in hata.h.
#include "hata.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "hata_launch.hpp"

namespace {

thread_local char g_msg[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HATA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_cus[kMaxDevices] = {0};

// Compute-unit count of the current device (cached).
int current_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HATA_ERR_HIP, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_cus[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    g_cus[dev] = cus > 0 ? cus : 1;
  }
  *out = g_cus[dev];
  return HATA_OK;
}

bool test_fail_launch() {
  const char* v = std::getenv("HATA_TEST_FAIL_LAUNCH");
  return v && v[0] == '1';
}

// Test hook: with HATA_TEST_FAIL_LAUNCH=1 every entry point reports a HIP
// failure after validating its arguments and before launching anything.
int pre_launch(const char* what) {
  if (test_fail_launch()) return fail(HATA_ERR_HIP, "%s: launch failure forced by HATA_TEST_FAIL_LAUNCH", what);
  return HATA_OK;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  return HATA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_dims(int d, int r) {
  if (d != 128) return fail(HATA_ERR_UNSUPPORTED, "head dim d=%d unsupported (only 128)", d);
  if (r != 32 && r != 64 && r != 128 && r != 256)
    return fail(HATA_ERR_UNSUPPORTED, "code width r=%d unsupported (32, 64, 128, 256)", r);
  return HATA_OK;
}

int check_heads(int B, int Hq, int Hkv) {
  if (B < 1) return fail(HATA_ERR_SHAPE, "B=%d must be >= 1", B);
  if (Hq < 1 || Hkv < 1) return fail(HATA_ERR_SHAPE, "Hq=%d, Hkv=%d must be >= 1", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(HATA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(HATA_ERR_UNSUPPORTED, "group size G=%d unsupported (1, 2, 4, 8)", G);
  if ((int64_t)B * Hkv > (1 << 24)) return fail(HATA_ERR_SHAPE, "B*Hkv=%lld too large", (long long)B * Hkv);
  return HATA_OK;
}

int check_len(int64_t cap, int64_t max_len) {
  if (cap < 1 || cap > (int64_t)1 << 30) return fail(HATA_ERR_SHAPE, "cap=%lld out of range [1, 2^30]", (long long)cap);
  if (max_len < 1 || max_len > cap)
    return fail(HATA_ERR_SHAPE, "max_len=%lld must lie in [1, cap=%lld]", (long long)max_len, (long long)cap);
  return HATA_OK;
}

int check_k(int k) {
  if (k < 1 || k > 4096) return fail(HATA_ERR_UNSUPPORTED, "budget k=%d outside [1, 4096]", k);
  return HATA_OK;
}

}  // namespace

extern "C" {

const char* hata_status_string(int status) {
  switch (status) {
    case HATA_OK: return "HATA_OK";
    case HATA_ERR_NULL: return "HATA_ERR_NULL: a required pointer is NULL";
    case HATA_ERR_SHAPE: return "HATA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case HATA_ERR_UNSUPPORTED: return "HATA_ERR_UNSUPPORTED: sizes outside the supported set";
    case HATA_ERR_ALIGN: return "HATA_ERR_ALIGN: misaligned pointer";
    case HATA_ERR_WORKSPACE: return "HATA_ERR_WORKSPACE: workspace missing or too small";
    case HATA_ERR_HIP: return "HATA_ERR_HIP: HIP runtime error";
    default: return "unknown hata_status";
  }
}

const char* hata_last_error_message(void) { return g_msg; }

int hata_version(void) { return 100; }

int hata_encode_append(const void* x, int64_t x_rows, int B, int H, int n_new, const float* W_H,
                       int Hkv, int d, int r, uint32_t* codes, int64_t cap, const int32_t* pos,
                       void* stream) {
  if (!x || !W_H || !codes) return fail(HATA_ERR_NULL, "encode_append: x, W_H and codes are required");
  int st = check_dims(d, r);
  if (st) return st;
  if (B < 1 || H < 1 || Hkv < 1) return fail(HATA_ERR_SHAPE, "encode_append: B=%d H=%d Hkv=%d", B, H, Hkv);
  if (H % Hkv != 0) return fail(HATA_ERR_SHAPE, "encode_append: H=%d not a multiple of Hkv=%d", H, Hkv);
  if (n_new < 0) return fail(HATA_ERR_SHAPE, "encode_append: n_new=%d < 0", n_new);
  if (x_rows < 1 || cap < 1) return fail(HATA_ERR_SHAPE, "encode_append: x_rows=%lld cap=%lld", (long long)x_rows, (long long)cap);
  if (!pos && ((int64_t)n_new > x_rows || (int64_t)n_new > cap))
    return fail(HATA_ERR_SHAPE, "encode_append: n_new=%d exceeds x_rows=%lld or cap=%lld", n_new, (long long)x_rows, (long long)cap);
  if ((int64_t)(H / Hkv) * n_new > ((int64_t)1 << 31) - 1) return fail(HATA_ERR_SHAPE, "encode_append: too many rows");
  if (!aligned(codes, 16)) return fail(HATA_ERR_ALIGN, "encode_append: codes must be 16-byte aligned");
  if (!aligned(x, 4)) return fail(HATA_ERR_ALIGN, "encode_append: x must be 4-byte aligned");
  if (n_new == 0) return HATA_OK;
  if ((st = pre_launch("encode_append"))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* xb = static_cast<const uint16_t*>(x);
  hipError_t e;
  // the matrix-core bulk encode is written for 128-bit codes; other widths
  // use the row kernel for every row count
  if (n_new >= hata::kBulkMinRows && r == 128)
    e = hata::launch_encode_bulk(xb, x_rows, B, H, Hkv, n_new, W_H, codes, cap, pos, 0, s);
  else
    e = hata::launch_encode_rows(xb, x_rows, B, H, Hkv, n_new, W_H, codes, cap, pos, 0, s, r);
  return check_launch(e, "encode_append launch");
}

int hata_hamming_scores(const uint32_t* q_codes, const uint32_t* k_codes, int B, int Hq, int Hkv,
                        int r, int64_t cap, const int32_t* seq_lens, int64_t max_len,
                        uint16_t* scores, void* stream) {
  if (!q_codes || !k_codes || !seq_lens || !scores) return fail(HATA_ERR_NULL, "hamming_scores: null pointer");
  int st = check_dims(128, r);
  if (st) return st;
  if ((st = check_heads(B, Hq, Hkv))) return st;
  if ((st = check_len(cap, max_len))) return st;
  if (!aligned(k_codes, 16) || !aligned(q_codes, 8) || !aligned(scores, 2))
    return fail(HATA_ERR_ALIGN, "hamming_scores: k_codes must be 16-byte aligned");
  if ((st = pre_launch("hamming_scores"))) return st;
  hipError_t e = hata::launch_hamming(q_codes, k_codes, B, Hq, Hkv, cap, seq_lens, max_len, scores,
                                      cap, reinterpret_cast<hipStream_t>(stream), r);
  return check_launch(e, "hamming_scores launch");
}

int hata_topk(const uint16_t* scores, int B, int Hkv, int64_t cap, const int32_t* seq_lens,
              int64_t max_len, int k, int max_score, int32_t* idx, void* ws, size_t ws_bytes,
              void* stream) {
  if (!scores || !seq_lens || !idx) return fail(HATA_ERR_NULL, "topk: null pointer");
  if (B < 1 || Hkv < 1) return fail(HATA_ERR_SHAPE, "topk: B=%d Hkv=%d", B, Hkv);
  int st = check_len(cap, max_len);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (max_score < 0 || max_score > 8 * 256)
    return fail(HATA_ERR_UNSUPPORTED, "topk: max_score=%d outside [0, 2048]", max_score);
  if (!aligned(scores, 2) || !aligned(idx, 4)) return fail(HATA_ERR_ALIGN, "topk: misaligned buffer");
  if ((st = pre_launch("topk"))) return st;
  // with a large enough workspace, long sequences are split over many workgroups
  void* scratch = (ws && ws_bytes >= hata::topk_scratch_bytes(B, Hkv, max_len, max_score)) ? ws : nullptr;
  hipError_t e = hata::launch_topk(scores, cap, B, Hkv, cap, seq_lens, k, max_score, idx,
                                   reinterpret_cast<hipStream_t>(stream), scratch, max_len);
  return check_launch(e, "topk launch");
}

int hata_sparse_decode(const void* q, const void* K, const void* V, int B, int Hq, int Hkv, int d,
                       int64_t cap, const int32_t* idx, int k, float scale, float* out, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!q || !K || !V || !idx || !out) return fail(HATA_ERR_NULL, "sparse_decode: null pointer");
  int st = check_dims(d, 128);
  if (st) return st;
  if ((st = check_heads(B, Hq, Hkv))) return st;
  if (cap < 1) return fail(HATA_ERR_SHAPE, "sparse_decode: cap=%lld", (long long)cap);
  if ((st = check_k(k))) return st;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16))
    return fail(HATA_ERR_ALIGN, "sparse_decode: q, K and V must be 16-byte aligned");
  const size_t need = hata_workspace_bytes(HATA_OP_SPARSE_DECODE, B, Hq, Hkv, d, 128, k, k);
  if (!ws || ws_bytes < need)
    return fail(HATA_ERR_WORKSPACE, "sparse_decode: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if ((st = pre_launch("sparse_decode"))) return st;
  hipError_t e = hata::launch_attention(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K),
                                        static_cast<const uint16_t*>(V), B, Hq, Hkv, cap, idx, k,
                                        nullptr, k, scale, out, static_cast<float*>(ws),
                                        reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "sparse_decode launch");
}

int hata_dense_decode(const void* q, const void* K, const void* V, int B, int Hq, int Hkv, int d,
                      int64_t cap, const int32_t* seq_lens, int64_t max_len, float scale,
                      float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !K || !V || !seq_lens || !out) return fail(HATA_ERR_NULL, "dense_decode: null pointer");
  int st = check_dims(d, 128);
  if (st) return st;
  if ((st = check_heads(B, Hq, Hkv))) return st;
  if ((st = check_len(cap, max_len))) return st;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16))
    return fail(HATA_ERR_ALIGN, "dense_decode: q, K and V must be 16-byte aligned");
  const size_t need = hata_workspace_bytes(HATA_OP_DENSE_DECODE, B, Hq, Hkv, d, 128, max_len, 1);
  if (!ws || ws_bytes < need)
    return fail(HATA_ERR_WORKSPACE, "dense_decode: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if ((st = pre_launch("dense_decode"))) return st;
  hipError_t e = hata::launch_attention(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K),
                                        static_cast<const uint16_t*>(V), B, Hq, Hkv, cap, nullptr, 0,
                                        seq_lens, max_len, scale, out, static_cast<float*>(ws),
                                        reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "dense_decode launch");
}

int hata_stream_read(const void* src, size_t bytes, uint64_t* sink, size_t sink_words, void* stream) {
  if (!src || !sink) return fail(HATA_ERR_NULL, "stream_read: null pointer");
  if (!aligned(src, 16) || bytes % 16 != 0)
    return fail(HATA_ERR_ALIGN, "stream_read: src must be 16-byte aligned and bytes a multiple of 16");
  if (sink_words < (size_t)hata::stream_read_blocks())
    return fail(HATA_ERR_WORKSPACE, "stream_read: sink of %d words needed, %zu given",
                hata::stream_read_blocks(), sink_words);
  int st = pre_launch("stream_read");
  if (st) return st;
  int cus = 0;
  if ((st = current_cus(&cus))) return st;
  // one workgroup per CU (as many as the sink holds)
  const int blocks = cus < hata::stream_read_blocks() ? cus : hata::stream_read_blocks();
  hipError_t e = hata::launch_stream_read(src, bytes, sink, blocks, reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "stream_read launch");
}

// noalloc: ws is ignored and the library's static scratch serves instead
static int decode_step_impl(const void* q, const void* K, const void* V, const float* W_H,
                            const float* W_Hk, uint32_t* codes, int B, int Hq, int Hkv, int d, int r,
                            int64_t cap, const int32_t* seq_lens, int64_t max_len, int k, float scale,
                            float* out, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream,
                            bool noalloc = false) {
  if (!q || !K || !V || !W_H || !W_Hk || !codes || !seq_lens || !out)
    return fail(HATA_ERR_NULL, "decode_step: null pointer");
  int st = check_dims(d, r);
  if (st) return st;
  if ((st = check_heads(B, Hq, Hkv))) return st;
  if ((st = check_len(cap, max_len))) return st;
  if ((st = check_k(k))) return st;
  if (!aligned(codes, 16) || !aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16))
    return fail(HATA_ERR_ALIGN, "decode_step: q, K, V and codes must be 16-byte aligned");
  int cus = 0;
  if ((st = current_cus(&cus))) return st;
  const hata::StepPlan p = hata::plan_decode_step(B, Hq, Hkv, max_len, k, cus, r);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* wsb = nullptr;
  if (noalloc) {
    // the static scratch stands in for the workspace: its flag and stamp
    // slots are cleared first (a fill kernel), since calls of other sizes
    // share them
    if (p.total > hata::kNoAllocScratchBytes)
      return fail(HATA_ERR_WORKSPACE, "decode_step_noalloc: these sizes need %zu bytes of scratch, above the "
                  "%zu-byte static scratch; use hata_decode_step with a workspace", p.total,
                  hata::kNoAllocScratchBytes);
    if ((st = pre_launch("decode_step_noalloc"))) return st;
    hipError_t e = hata::noalloc_scratch(&wsb);
    if (e != hipSuccess) return hip_fail(e, "decode_step_noalloc: hipGetSymbolAddress");
    if (p.fused) {
      e = hata::launch_fill_zero(wsb, p.off_win, s);
      if (e != hipSuccess) return hip_fail(e, "decode_step_noalloc: clearing the scratch flags");
    }
  } else {
    if (!ws || ws_bytes < p.total)
      return fail(HATA_ERR_WORKSPACE, "decode_step: workspace of %zu bytes needed, %zu given", p.total, ws_bytes);
    if ((st = pre_launch("decode_step"))) return st;
    wsb = static_cast<unsigned char*>(ws);
  }
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* Kb = static_cast<const uint16_t*>(K);
  const auto* Vb = static_cast<const uint16_t*>(V);
  if (p.fused) {
    hipError_t e = hata::launch_decode_step(p, qb, Kb, Vb, W_H, W_Hk, codes, B, Hq, Hkv, cap, seq_lens,
                                            k, scale, out, idx_out, wsb, s);
    return check_launch(e, "decode_step launch");
  }
  // Staged steps: the per-unit scores do not fit on chip at this shape.
  const int G = Hq / Hkv;
  auto* qc = reinterpret_cast<uint32_t*>(wsb + p.off_qc);
  auto* sc = reinterpret_cast<uint16_t*>(wsb + p.off_scores);
  auto* part = reinterpret_cast<float*>(wsb + p.off_attn);
  // the kept list goes to idx_out, or to the workspace when it is NULL
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(wsb + p.off_idx);
  auto* hist = reinterpret_cast<uint32_t*>(wsb + p.off_topk);  // unit histograms, filled by the scan
  hipError_t e = hata::launch_fill_zero(hist, (size_t)B * Hkv * (G * r + 1) * 4, s);
  if (e == hipSuccess) e = hata::launch_encode_rows(qb, 1, B, Hq, Hkv, 1, W_H, qc, 1, nullptr, 0, s, r);
  if (e == hipSuccess)  // key append at row seq_lens[b] - 1
    e = hata::launch_encode_rows(Kb, cap, B, Hkv, Hkv, 1, W_Hk, codes, cap, seq_lens, -1, s, r);
  if (e == hipSuccess)
    e = hata::launch_hamming(qc, codes, B, Hq, Hkv, cap, seq_lens, max_len, sc, max_len, s, r, nullptr, hist);
  if (e == hipSuccess)
    e = hata::launch_topk_after_hamming(sc, max_len, B, Hkv, cap, seq_lens, k, G * r, idx, s, wsb + p.off_topk,
                                        max_len);
  if (e == hipSuccess)
    e = hata::launch_attention(qb, Kb, Vb, B, Hq, Hkv, cap, idx, k, nullptr, k, scale, out, part, s);
  return check_launch(e, "decode_step (staged) launch");
}

namespace {
// workspace of the paged step: query codes, scores, kept indices, attention records
struct PagedPlan {
  size_t qc = 0, sc = 0, idx = 0, attn = 0, topk = 0, total = 0;
};
PagedPlan plan_paged(int B, int Hq, int Hkv, int64_t max_len, int k, int r) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  PagedPlan p;
  const size_t U = (size_t)B * Hkv;
  size_t off = 0;
  p.qc = off;   off = al(off + (size_t)B * Hq * ((r + 31) / 32) * 4);
  p.sc = off;   off = al(off + U * (size_t)max_len * 2);
  p.idx = off;  off = al(off + U * (size_t)k * 4);
  p.attn = off; off = al(off + hata::attn_part_floats(B, Hkv, Hq / Hkv, k) * 4);
  p.topk = off; off = al(off + hata::topk_scratch_bytes(B, Hkv, max_len, (Hq / Hkv) * r));
  p.total = off;
  return p;
}
}  // namespace

int hata_decode_step_paged(const void* q, const void* K_pool, const void* V_pool, const float* W_H,
                           uint32_t* code_pool, const int32_t* block_table, int max_pages, int num_pages,
                           int page_rows, int B, int Hq, int Hkv, int d, int r, const int32_t* seq_lens,
                           int64_t max_len, int k, float scale, float* out, int32_t* idx_out, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!q || !K_pool || !V_pool || !W_H || !code_pool || !block_table || !seq_lens || !out)
    return fail(HATA_ERR_NULL, "decode_step_paged: null pointer");
  int st = check_dims(d, r);
  if (st) return st;
  if ((st = check_heads(B, Hq, Hkv))) return st;
  if ((st = check_k(k))) return st;
  if (page_rows < 16 || page_rows > 65536 || (page_rows & (page_rows - 1)) != 0)
    return fail(HATA_ERR_UNSUPPORTED, "decode_step_paged: page_rows=%d not a power of two in [16, 65536]",
                page_rows);
  if (max_pages < 1 || num_pages < 1)
    return fail(HATA_ERR_SHAPE, "decode_step_paged: max_pages=%d, num_pages=%d must be >= 1", max_pages, num_pages);
  const int64_t cap = (int64_t)max_pages * page_rows;
  if ((st = check_len(cap, max_len))) return st;
  if (!aligned(code_pool, 16) || !aligned(q, 16) || !aligned(K_pool, 16) || !aligned(V_pool, 16))
    return fail(HATA_ERR_ALIGN, "decode_step_paged: q, K_pool, V_pool and code_pool must be 16-byte aligned");
  if (!aligned(block_table, 4)) return fail(HATA_ERR_ALIGN, "decode_step_paged: block_table must be 4-byte aligned");
  // workspace: the fused step's area, then the staged steps' area
  int cus = 0;
  if ((st = current_cus(&cus))) return st;
  const hata::StepPlan sp = hata::plan_decode_step(B, Hq, Hkv, max_len, k, cus, r);
  const PagedPlan p = plan_paged(B, Hq, Hkv, max_len, k, r);
  const size_t need = sp.total + p.total;
  if (!ws || ws_bytes < need)
    return fail(HATA_ERR_WORKSPACE, "decode_step_paged: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if ((st = pre_launch("decode_step_paged"))) return st;
  hata::PageMap pm;
  pm.bt = block_table;
  pm.max_pages = max_pages;
  pm.num_pages = num_pages;
  int lg = 0;
  while ((1 << lg) < page_rows) ++lg;
  pm.log2P = lg;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hata::decode_step_paged_fusable(sp, page_rows)) {
    hipError_t e = hata::launch_decode_step_paged(sp, static_cast<const uint16_t*>(q),
                                                  static_cast<const uint16_t*>(K_pool),
                                                  static_cast<const uint16_t*>(V_pool), W_H, code_pool, pm, Hq, Hkv,
                                                  seq_lens, k, scale, out, idx_out, static_cast<unsigned char*>(ws), s);
    return check_launch(e, "decode_step_paged launch");
  }
  auto* wsb = static_cast<unsigned char*>(ws) + sp.total;
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* Kb = static_cast<const uint16_t*>(K_pool);
  const auto* Vb = static_cast<const uint16_t*>(V_pool);
  const int G = Hq / Hkv;
  auto* qc = reinterpret_cast<uint32_t*>(wsb + p.qc);
  auto* sc = reinterpret_cast<uint16_t*>(wsb + p.sc);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(wsb + p.idx);
  auto* part = reinterpret_cast<float*>(wsb + p.attn);
  // the top-k scratch starts with the unit histograms, which the Hamming
  // scan fills
  auto* hist = reinterpret_cast<uint32_t*>(wsb + p.topk);
  hipError_t e = hata::launch_fill_zero(hist, (size_t)B * Hkv * (G * r + 1) * 4, s);
  if (e == hipSuccess) e = hata::launch_encode_rows(qb, 1, B, Hq, Hkv, 1, W_H, qc, 1, nullptr, 0, s, r);
  if (e == hipSuccess)  // key append at logical row seq_lens[b] - 1, through the page table
    e = hata::launch_encode_rows(Kb, cap, B, Hkv, Hkv, 1, W_H, code_pool, cap, seq_lens, -1, s, r, &pm);
  if (e == hipSuccess)
    e = hata::launch_hamming(qc, code_pool, B, Hq, Hkv, cap, seq_lens, max_len, sc, max_len, s, r, &pm, hist);
  if (e == hipSuccess)
    e = hata::launch_topk_after_hamming(sc, max_len, B, Hkv, cap, seq_lens, k, G * r, idx, s, wsb + p.topk,
                                        max_len);
  if (e == hipSuccess)
    e = hata::launch_attention(qb, Kb, Vb, B, Hq, Hkv, cap, idx, k, nullptr, k, scale, out, part, s, &pm);
  return check_launch(e, "decode_step_paged launch");
}

int hata_decode_step(const void* q, const void* K, const void* V, const float* W_H, uint32_t* codes,
                     int B, int Hq, int Hkv, int d, int r, int64_t cap, const int32_t* seq_lens,
                     int64_t max_len, int k, float scale, float* out, int32_t* idx_out, void* ws,
                     size_t ws_bytes, void* stream) {
  return decode_step_impl(q, K, V, W_H, W_H, codes, B, Hq, Hkv, d, r, cap, seq_lens, max_len, k, scale,
                          out, idx_out, ws, ws_bytes, stream);
}

int hata_decode_step_noalloc(const void* q, const void* K, const void* V, const float* W_H, uint32_t* codes,
                             int B, int Hq, int Hkv, int d, int r, int64_t cap, const int32_t* seq_lens,
                             int64_t max_len, int k, float scale, float* out, int32_t* idx_out, void* stream) {
  return decode_step_impl(q, K, V, W_H, W_H, codes, B, Hq, Hkv, d, r, cap, seq_lens, max_len, k, scale,
                          out, idx_out, nullptr, 0, stream, true);
}

int hata_decode_step_qk(const void* q, const void* K, const void* V, const float* W_Hq,
                        const float* W_Hk, uint32_t* codes, int B, int Hq, int Hkv, int d, int r,
                        int64_t cap, const int32_t* seq_lens, int64_t max_len, int k, float scale,
                        float* out, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  return decode_step_impl(q, K, V, W_Hq, W_Hk, codes, B, Hq, Hkv, d, r, cap, seq_lens, max_len, k, scale,
                          out, idx_out, ws, ws_bytes, stream);
}

int hata_hash_labels(const void* q, const void* k, const int32_t* q_pos, int J, int n, int d,
                     int pos_permille, float s_max, float s_min, float* labels, void* stream) {
  if (!q || !k || !q_pos || !labels) return fail(HATA_ERR_NULL, "hash_labels: null pointer");
  if (d != 128) return fail(HATA_ERR_UNSUPPORTED, "hash_labels: d=%d unsupported (only 128)", d);
  if (J < 1 || n < 1) return fail(HATA_ERR_SHAPE, "hash_labels: J=%d n=%d must be >= 1", J, n);
  if (n > hata::kMaxLabelKeys)
    return fail(HATA_ERR_UNSUPPORTED, "hash_labels: n=%d above %d keys", n, hata::kMaxLabelKeys);
  if (pos_permille < 1 || pos_permille > 1000)
    return fail(HATA_ERR_SHAPE, "hash_labels: pos_permille=%d outside [1, 1000]", pos_permille);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(labels, 4))
    return fail(HATA_ERR_ALIGN, "hash_labels: q and k must be 16-byte aligned, labels 4-byte aligned");
  int st = pre_launch("hash_labels");
  if (st) return st;
  hipError_t e = hata::launch_hash_labels(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), q_pos,
                                          J, n, pos_permille, s_max, s_min, labels,
                                          reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "hash_labels launch");
}

int hata_prefill(const void* q, const void* K, const void* V, const float* W_H, uint32_t* codes, int B, int Hq,
                 int Hkv, int d, int r, int64_t q_rows, int64_t cap, const int32_t* seq_lens, int64_t max_len,
                 float scale, float* out, void* stream) {
  if (!q || !K || !V || !W_H || !codes || !seq_lens || !out)
    return fail(HATA_ERR_NULL, "prefill: q, K, V, W_H, codes, seq_lens and out are required");
  int st = check_dims(d, r);
  if (st) return st;
  st = check_heads(B, Hq, Hkv);
  if (st) return st;
  st = check_len(cap, max_len);
  if (st) return st;
  if (q_rows < max_len)
    return fail(HATA_ERR_SHAPE, "prefill: q_rows=%lld below max_len=%lld", (long long)q_rows, (long long)max_len);
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16))
    return fail(HATA_ERR_ALIGN, "prefill: q, K, V and out must be 16-byte aligned");
  if (!aligned(codes, 8) || !aligned(W_H, 4) || !aligned(seq_lens, 4))
    return fail(HATA_ERR_ALIGN, "prefill: codes must be 8-byte, W_H and seq_lens 4-byte aligned");
  const int G = Hq / Hkv;
  const int64_t blocks = (max_len + hata::prefill_positions_per_block(G) - 1) / hata::prefill_positions_per_block(G);
  if (blocks * B * Hkv > ((int64_t)1 << 31) - 1)
    return fail(HATA_ERR_SHAPE, "prefill: grid of %lld workgroups too large", (long long)(blocks * B * Hkv));
  st = pre_launch("prefill");
  if (st) return st;
  hipError_t e = hata::launch_prefill(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K),
                                      static_cast<const uint16_t*>(V), W_H, codes, B, Hq, Hkv, q_rows, cap, seq_lens,
                                      (int)max_len, scale, out, r, reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "prefill launch");
}

int hata_prefill_paged(const void* q, const void* K_pool, const void* V_pool, const float* W_H,
                       uint32_t* code_pool, const int32_t* block_table, int max_pages, int num_pages, int page_rows,
                       int B, int Hq, int Hkv, int d, int r, int64_t q_rows, const int32_t* seq_lens,
                       int64_t max_len, float scale, float* out, void* stream) {
  if (!q || !K_pool || !V_pool || !W_H || !code_pool || !block_table || !seq_lens || !out)
    return fail(HATA_ERR_NULL, "prefill_paged: null pointer");
  int st = check_dims(d, r);
  if (st) return st;
  if ((st = check_heads(B, Hq, Hkv))) return st;
  if (page_rows < 16 || page_rows > 65536 || (page_rows & (page_rows - 1)) != 0)
    return fail(HATA_ERR_UNSUPPORTED, "prefill_paged: page_rows=%d not a power of two in [16, 65536]", page_rows);
  if (max_pages < 1 || num_pages < 1)
    return fail(HATA_ERR_SHAPE, "prefill_paged: max_pages=%d, num_pages=%d must be >= 1", max_pages, num_pages);
  const int64_t cap = (int64_t)max_pages * page_rows;
  if ((st = check_len(cap, max_len))) return st;
  if (q_rows < max_len)
    return fail(HATA_ERR_SHAPE, "prefill_paged: q_rows=%lld below max_len=%lld", (long long)q_rows,
                (long long)max_len);
  if (!aligned(q, 16) || !aligned(K_pool, 16) || !aligned(V_pool, 16) || !aligned(out, 16))
    return fail(HATA_ERR_ALIGN, "prefill_paged: q, K_pool, V_pool and out must be 16-byte aligned");
  if (!aligned(code_pool, 8) || !aligned(W_H, 4) || !aligned(seq_lens, 4) || !aligned(block_table, 4))
    return fail(HATA_ERR_ALIGN, "prefill_paged: code_pool must be 8-byte, W_H, seq_lens and block_table 4-byte aligned");
  const int G = Hq / Hkv;
  const int64_t blocks = (max_len + hata::prefill_positions_per_block(G) - 1) / hata::prefill_positions_per_block(G);
  if (blocks * B * Hkv > ((int64_t)1 << 31) - 1)
    return fail(HATA_ERR_SHAPE, "prefill_paged: grid of %lld workgroups too large", (long long)(blocks * B * Hkv));
  if ((st = pre_launch("prefill_paged"))) return st;
  hata::PageMap pm;
  pm.bt = block_table;
  pm.max_pages = max_pages;
  pm.num_pages = num_pages;
  int lg = 0;
  while ((1 << lg) < page_rows) ++lg;
  pm.log2P = lg;
  hipError_t e = hata::launch_prefill(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K_pool),
                                      static_cast<const uint16_t*>(V_pool), W_H, code_pool, B, Hq, Hkv, q_rows, cap,
                                      seq_lens, (int)max_len, scale, out, r, reinterpret_cast<hipStream_t>(stream),
                                      &pm);
  return check_launch(e, "prefill_paged launch");
}

size_t hata_hash_train_workspace_bytes(int J, int n, int d, int r) {
  if (J < 1 || n < 1 || d != 128 || r < 32 || r > 256 || r % 32 != 0) return 0;
  return hata::plan_train(J, n, r).total;
}

int hata_hash_train_step(const void* q, const void* k, const int32_t* q_pos, const float* labels, int J, int n,
                         int d, int r, float sigma, float eps, float eta, float lam, float lr, float* W,
                         float* grad, float* loss, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !q_pos || !labels || !W || !loss) return fail(HATA_ERR_NULL, "hash_train_step: null pointer");
  if (d != 128) return fail(HATA_ERR_UNSUPPORTED, "hash_train_step: d=%d unsupported (only 128)", d);
  if (r < 32 || r > 256 || r % 32 != 0)
    return fail(HATA_ERR_UNSUPPORTED, "hash_train_step: r=%d unsupported (multiples of 32 up to 256)", r);
  if (J < 1 || n < 1 || (int64_t)J * n > ((int64_t)1 << 31))
    return fail(HATA_ERR_SHAPE, "hash_train_step: J=%d n=%d", J, n);
  if (!aligned(q, 4) || !aligned(k, 4) || !aligned(labels, 4) || !aligned(W, 4))
    return fail(HATA_ERR_ALIGN, "hash_train_step: misaligned buffer");
  const hata::TrainPlan p = hata::plan_train(J, n, r);
  if (!ws || ws_bytes < p.total)
    return fail(HATA_ERR_WORKSPACE, "hash_train_step: workspace of %zu bytes needed, %zu given", p.total, ws_bytes);
  int st = pre_launch("hash_train_step");
  if (st) return st;
  hipError_t e = hata::launch_hash_train_step(p, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                              q_pos, labels, J, n, r, sigma, eps, eta, lam, lr, W, grad, loss,
                                              static_cast<unsigned char*>(ws), reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "hash_train_step launch");
}

size_t hata_workspace_bytes(int op, int B, int Hq, int Hkv, int d, int r, int64_t max_len, int k) {
  (void)d;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_len < 1 || k < 1) return 0;
  if (r != 32 && r != 64 && r != 128 && r != 256) return 0;
  const int G = Hq / Hkv;
  switch (op) {
    case HATA_OP_TOPK:
      return hata::topk_scratch_bytes(B, Hkv, max_len, G * r);
    case HATA_OP_SPARSE_DECODE:
      return hata::attn_part_floats(B, Hkv, G, k) * sizeof(float);
    case HATA_OP_DENSE_DECODE:
      return hata::attn_part_floats(B, Hkv, G, max_len) * sizeof(float);
    case HATA_OP_DECODE_STEP: {
      int cus = 0;
      if (current_cus(&cus) != HATA_OK) return 0;
      return hata::plan_decode_step(B, Hq, Hkv, max_len, k, cus, r).total;
    }
    case HATA_OP_DECODE_STEP_PAGED: {
      int cus = 0;
      if (current_cus(&cus) != HATA_OK) return 0;
      return hata::plan_decode_step(B, Hq, Hkv, max_len, k, cus, r).total + plan_paged(B, Hq, Hkv, max_len, k, r).total;
    }
    default:
      return 0;
  }
}

int hata_workspace_reset(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return fail(HATA_ERR_NULL, "workspace_reset: ws is NULL");
  if (ws_bytes == 0) return HATA_OK;
  if (!aligned(ws, 4)) return fail(HATA_ERR_ALIGN, "workspace_reset: ws must be 4-byte aligned");
  if (int st = pre_launch("workspace_reset")) return st;
  hipError_t e = hata::launch_fill_zero(ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "workspace_reset launch");
}

int hata_workspace_set_spin_limit(void* ws, size_t ws_bytes, uint32_t polls, void* stream) {
  if (!ws) return fail(HATA_ERR_NULL, "workspace_set_spin_limit: ws is NULL");
  if (ws_bytes < 8) return fail(HATA_ERR_WORKSPACE, "workspace_set_spin_limit: workspace too small");
  if (!aligned(ws, 4)) return fail(HATA_ERR_ALIGN, "workspace_set_spin_limit: ws must be 4-byte aligned");
  if (int st = pre_launch("workspace_set_spin_limit")) return st;
  hipError_t e = hata::launch_set_word(static_cast<uint32_t*>(ws) + 1, polls, reinterpret_cast<hipStream_t>(stream));
  return check_launch(e, "workspace_set_spin_limit launch");
}

int hata_workspace_check(const void* ws, size_t ws_bytes, int* err_out, void* stream) {
  if (!ws || !err_out) return fail(HATA_ERR_NULL, "workspace_check: null pointer");
  if (ws_bytes < 4) return fail(HATA_ERR_WORKSPACE, "workspace_check: workspace too small");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t v = 0;
  e = hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  *err_out = (int)v;
  return HATA_OK;
}

}  // extern "C"
