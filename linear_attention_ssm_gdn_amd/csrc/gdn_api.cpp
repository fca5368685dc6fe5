// gdn_api.cpp -- the C ABI of libgdn: argument validation, page layouts and
// kernel launches.  Every check here runs on the host before anything is
// launched, so a bad argument returns GDN_ERR_ARG without touching the GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/gdn.h"
#include "gdn_kernels.h"

#define GDN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

int64_t c_conv(const gdn_dims* d) { return 2 * (int64_t)d->h_k * d->d_k + (int64_t)d->h_v * d->d_v; }

size_t elem_size(int32_t dt) { return dt == GDN_BF16 ? 2 : 4; }

bool dtype_ok(int32_t dt) { return dt == GDN_F32 || dt == GDN_BF16; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Structural checks shared by every entry point.
int32_t check_dims(const gdn_dims* d) {
    if (!d) return GDN_ERR_ARG;
    if (d->h_k <= 0 || d->h_v <= 0 || d->h_v % d->h_k != 0) return GDN_ERR_ARG;
    if (d->d_k <= 0 || d->d_v <= 0 || d->conv_w <= 1 || d->n_spec < 0) return GDN_ERR_ARG;
    if (!dtype_ok(d->act_dtype) || !dtype_ok(d->state_dtype)) return GDN_ERR_ARG;
    if (!std::isfinite(d->scale) || !std::isfinite(d->l2_eps) || d->l2_eps < 0.0f) return GDN_ERR_ARG;
    if ((int64_t)d->h_k * d->d_k > (1 << 24) || (int64_t)d->h_v * d->d_v > (1 << 24)) return GDN_ERR_ARG;
    if (d->conv_w != 4) return GDN_ERR_UNSUPPORTED;
    if (!gdn::seq_supported(d->d_k, d->d_v)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

int32_t check_params(const gdn_params* p) {
    if (!p || !p->conv_w || !p->a_log || !p->dt_bias) return GDN_ERR_ARG;
    return GDN_OK;
}

int32_t check_batch(const gdn_batch* b) {
    if (!b || b->n_seqs < 0 || b->max_seqlen < 0 || b->n_rows < 0) return GDN_ERR_ARG;
    if (b->n_rows > INT32_MAX) return GDN_ERR_ARG;
    if (b->n_seqs > 0 && (!b->cu_seqlens || !b->page_idx)) return GDN_ERR_ARG;
    return GDN_OK;
}

int32_t check_conv_pool(const gdn_dims* d, const gdn_conv_pool& c, int32_t min_rows, bool need_sync) {
    if (!c.base || c.rows < min_rows || c.n_pages < 0) return GDN_ERR_ARG;
    if (c.page_stride < (int64_t)c.rows * c_conv(d)) return GDN_ERR_ARG;
    if (need_sync && !c.sync) return GDN_ERR_ARG;
    return GDN_OK;
}

int32_t check_state_pool(const gdn_dims* d, const gdn_state_pool& s) {
    const size_t es = elem_size(d->state_dtype);
    if (!s.base || s.n_pages < 0) return GDN_ERR_ARG;
    if (s.page_stride < (int64_t)d->h_v * d->d_k * d->d_v) return GDN_ERR_ARG;
    if ((s.page_stride * (int64_t)es) % 16 != 0 || !aligned(s.base, 16)) return GDN_ERR_ARG;
    return GDN_OK;
}

int32_t from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Shared validation of the sequence entry points (token by token, chunked).
int32_t check_sequence_call(const gdn_dims* dims, const gdn_params* params, const void* x,
                            int64_t x_stride, const void* a, const void* b, int64_t ab_stride,
                            const gdn_batch* batch, const gdn_conv_pool& conv,
                            const gdn_state_pool& state, const float* o, bool need_sync = true) {
    int32_t st;
    if ((st = check_dims(dims)) != GDN_OK) return st;
    if ((st = check_params(params)) != GDN_OK) return st;
    if ((st = check_batch(batch)) != GDN_OK) return st;
    if (batch->n_seqs == 0) return GDN_OK;
    if ((st = check_conv_pool(dims, conv, dims->conv_w - 1, need_sync)) != GDN_OK) return st;
    if ((st = check_state_pool(dims, state)) != GDN_OK) return st;
    if (batch->n_rows > 0 && (!x || !a || !b || !o)) return GDN_ERR_ARG;
    if (x_stride < c_conv(dims) || ab_stride < dims->h_v) return GDN_ERR_ARG;
    return GDN_OK;
}

gdn::SeqArgs seq_args(const gdn_dims* dims, const gdn_params* params, const void* x, int64_t x_stride,
                      const void* a, const void* b, int64_t ab_stride, const gdn_batch* batch,
                      const gdn_conv_pool& conv, const gdn_state_pool& state, float* o, int32_t* err) {
    gdn::SeqArgs A{};
    A.x = x; A.x_stride = x_stride; A.a = a; A.b = b; A.ab_stride = ab_stride; A.n_rows = batch->n_rows;
    A.cu = batch->cu_seqlens; A.page_idx = batch->page_idx; A.has_init = batch->has_init; A.n_seqs = batch->n_seqs;
    A.conv_w = params->conv_w; A.a_log = params->a_log; A.dt_bias = params->dt_bias;
    A.conv_base = conv.base; A.conv_page_stride = conv.page_stride; A.conv_n_pages = conv.n_pages; A.sync = conv.sync;
    A.state = state.base; A.state_page_stride = state.page_stride; A.state_n_pages = state.n_pages;
    A.o = o; A.err = err; A.h_k = dims->h_k; A.h_v = dims->h_v; A.d_v = dims->d_v;
    A.scale = dims->scale; A.eps = dims->l2_eps;
    return A;
}

// Validation of a verify call (dims and params already checked); fills *L.
int32_t check_verify_call(const gdn_dims* dims, int32_t layout, const void* x, int64_t x_stride, const void* a,
                          const void* b, int64_t ab_stride, int32_t n_req, int32_t n_cand, const int32_t* req_page,
                          const int32_t* num_accepted, const uint8_t* step_parity, const void* pages,
                          int64_t page_bytes, int32_t n_pages, const gdn_conv_pool& conv, const float* o,
                          gdn_spec_layout* L) {
    int32_t st;
    if ((st = gdn_spec_page_layout(dims, layout, L)) != GDN_OK) return st;
    if (n_req < 0 || n_cand < 0 || n_cand > dims->n_spec + 1) return GDN_ERR_ARG;
    if (n_req == 0) return GDN_OK;
    if (!req_page || !num_accepted || !step_parity || !pages || n_pages < 0) return GDN_ERR_ARG;
    if (page_bytes < (int64_t)L->page_bytes || page_bytes % 256 != 0 || !aligned(pages, 256)) return GDN_ERR_ARG;
    if ((st = check_conv_pool(dims, conv, dims->conv_w - 1 + dims->n_spec, true)) != GDN_OK) return st;
    if (n_cand > 0 && (!x || !a || !b || !o)) return GDN_ERR_ARG;
    if (n_cand > 0 && (x_stride < c_conv(dims) || ab_stride < dims->h_v)) return GDN_ERR_ARG;
    return GDN_OK;
}

gdn::VerifyArgs verify_args(const gdn_dims* dims, const gdn_params* params, const gdn_spec_layout& L, const void* x,
                            int64_t x_stride, const void* a, const void* b, int64_t ab_stride, int32_t n_req,
                            int32_t n_cand, const int32_t* req_page, const int32_t* num_accepted,
                            const uint8_t* step_parity, void* pages, int64_t page_bytes, int32_t n_pages,
                            const gdn_conv_pool& conv, float* o, int32_t* err) {
    gdn::VerifyArgs A{};
    A.x = x; A.x_stride = x_stride; A.a = a; A.b = b; A.ab_stride = ab_stride;
    A.n_req = n_req; A.n_cand = n_cand;
    A.req_page = req_page; A.num_accepted = num_accepted; A.step_parity = step_parity;
    A.pages = static_cast<uint8_t*>(pages); A.page_bytes = page_bytes; A.n_pages = n_pages;
    A.header_off = (int64_t)L.header_off; A.state_off = (int64_t)L.state_off;
    A.record_off = (int64_t)L.record_off; A.record_row_bytes = (int64_t)L.record_row_bytes;
    A.conv_w = params->conv_w; A.a_log = params->a_log; A.dt_bias = params->dt_bias;
    A.conv_base = conv.base; A.conv_page_stride = conv.page_stride; A.conv_n_pages = conv.n_pages; A.sync = conv.sync;
    A.o = o; A.err = err; A.h_k = dims->h_k; A.h_v = dims->h_v; A.d_v = dims->d_v; A.n_spec = dims->n_spec;
    A.scale = dims->scale; A.eps = dims->l2_eps;
    return A;
}

}  // namespace

namespace gdn {
// Validation and argument block of a token-by-token call whose sync words
// the caller does not supply (conv.sync may be NULL): used by the entry
// point that keeps them in the library's own device array.
int32_t seq_call_args_nosync(const gdn_dims* dims, const gdn_params* params, const void* x, int64_t x_stride,
                             const void* a, const void* b, int64_t ab_stride, const gdn_batch* batch,
                             const gdn_conv_pool& conv, const gdn_state_pool& state, float* o, int32_t* err,
                             SeqArgs* out) {
    const int32_t st = check_sequence_call(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o, false);
    if (st != GDN_OK || batch->n_seqs == 0) return st;
    *out = seq_args(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o, err);
    return GDN_OK;
}
}  // namespace gdn

GDN_EXPORT int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

GDN_EXPORT const char* gdn_status_str(int32_t status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

GDN_EXPORT int32_t gdn_spec_page_layout(const gdn_dims* dims, int32_t layout, gdn_spec_layout* out) {
    int32_t st = check_dims(dims);
    if (st != GDN_OK) return st;
    if (!out || (layout != GDN_SPEC_ONEPAGE && layout != GDN_SPEC_SLOTS)) return GDN_ERR_ARG;
    if (dims->n_spec + 1 > 16) return GDN_ERR_UNSUPPORTED;
    const size_t head = (size_t)dims->d_k * dims->d_v * elem_size(dims->state_dtype);
    const size_t rows = (size_t)dims->n_spec + 1;
    out->header_off = 0;
    out->state_off = round_up(sizeof(gdn_spec_header));
    if (layout == GDN_SPEC_ONEPAGE) {
        out->record_row_bytes = ((size_t)c_conv(dims) + 2 * (size_t)dims->h_v) * sizeof(float);
        out->record_off = round_up(out->state_off + (size_t)dims->h_v * head);
        out->page_bytes = round_up(out->record_off + 2 * rows * out->record_row_bytes);
    } else {
        out->record_row_bytes = 0;
        out->record_off = 0;
        out->page_bytes = round_up(out->state_off + rows * (size_t)dims->h_v * head);
    }
    return GDN_OK;
}

GDN_EXPORT int32_t gdn_chunked_workspace_bytes(const gdn_dims* dims, int32_t n_seqs, int64_t n_rows,
                                               int32_t chunk, size_t* out_bytes) {
    int32_t st = check_dims(dims);
    if (st != GDN_OK) return st;
    if (!out_bytes || n_seqs < 0 || n_rows < 0 || chunk <= 0) return GDN_ERR_ARG;
    if (!gdn::chunked_supported(dims->d_k, dims->d_v, chunk)) return GDN_ERR_UNSUPPORTED;
    *out_bytes = gdn::chunked_workspace_bytes(dims->h_k, dims->h_v, n_seqs, n_rows);
    return GDN_OK;
}

GDN_EXPORT int32_t gdn_conv_update(const gdn_dims* dims, const void* conv_w, const void* x, int64_t x_stride,
                                   const gdn_batch* batch, gdn_conv_pool conv, int32_t activation, void* y,
                                   int32_t y_dtype, int64_t y_stride, int32_t* err, void* stream) {
    int32_t st;
    if ((st = check_dims(dims)) != GDN_OK) return st;
    if ((st = check_batch(batch)) != GDN_OK) return st;
    if (!conv_w || !dtype_ok(y_dtype) || (activation != 0 && activation != 1)) return GDN_ERR_ARG;
    if (batch->n_seqs == 0) return GDN_OK;
    if ((st = check_conv_pool(dims, conv, dims->conv_w - 1, false)) != GDN_OK) return st;
    const int64_t C = c_conv(dims);
    if (batch->n_rows > 0 && (!x || !y)) return GDN_ERR_ARG;
    if (x_stride < C || y_stride < C) return GDN_ERR_ARG;
    gdn::ConvArgs A{};
    A.x = x; A.x_stride = x_stride; A.n_rows = batch->n_rows;
    A.cu = batch->cu_seqlens; A.page_idx = batch->page_idx; A.has_init = batch->has_init; A.n_seqs = batch->n_seqs;
    A.conv_w = conv_w;
    A.conv_base = conv.base; A.conv_page_stride = conv.page_stride; A.conv_n_pages = conv.n_pages;
    A.y = y; A.y_stride = y_stride; A.err = err; A.C = (int32_t)C; A.activation = activation;
    return from_hip(gdn::launch_conv(A, dims->act_dtype, y_dtype, batch->max_seqlen, (hipStream_t)stream));
}

GDN_EXPORT int32_t gdn_recurrent_seq(const gdn_dims* dims, const gdn_params* params, const void* x,
                                     int64_t x_stride, const void* a, const void* b, int64_t ab_stride,
                                     const gdn_batch* batch, gdn_conv_pool conv, gdn_state_pool state, float* o,
                                     int32_t* err, void* stream) {
    int32_t st = check_sequence_call(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o);
    if (st != GDN_OK || batch->n_seqs == 0) return st;
    const gdn::SeqArgs A = seq_args(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o, err);
    return from_hip(gdn::launch_seq(A, dims->d_k, dims->act_dtype, dims->state_dtype, batch->max_seqlen,
                                    (hipStream_t)stream));
}

GDN_EXPORT int32_t gdn_chunked_prefill(const gdn_dims* dims, const gdn_params* params, const void* x,
                                       int64_t x_stride, const void* a, const void* b, int64_t ab_stride,
                                       const gdn_batch* batch, gdn_conv_pool conv, gdn_state_pool state, float* o,
                                       int32_t chunk, void* workspace, size_t ws_bytes, int32_t* err,
                                       void* stream) {
    int32_t st = check_sequence_call(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o);
    if (st != GDN_OK) return st;
    if (chunk <= 0) return GDN_ERR_ARG;
    if (!gdn::chunked_supported(dims->d_k, dims->d_v, chunk)) return GDN_ERR_UNSUPPORTED;
    // x and conv-window rows are read, and o rows written, as 16-byte vectors
    const int64_t vec = dims->act_dtype == GDN_BF16 ? 8 : 4;
    if (batch->n_seqs > 0 && (!aligned(x, 16) || x_stride % vec != 0 || !aligned(conv.base, 16) ||
                              conv.page_stride % vec != 0 || !aligned(o, 16)))
        return GDN_ERR_ARG;
    // one chunk's x rows and output rows are addressed with 32-bit offsets
    if (x_stride > (int64_t)1 << 24 || (int64_t)dims->h_v * dims->d_v > (int64_t)1 << 24) return GDN_ERR_ARG;
    size_t need = 0;
    if ((st = gdn_chunked_workspace_bytes(dims, batch->n_seqs, batch->n_rows, chunk, &need)) != GDN_OK) return st;
    if (ws_bytes < need || (need > 0 && (!workspace || !aligned(workspace, 256)))) return GDN_ERR_ARG;
    if (batch->n_seqs == 0) return GDN_OK;
    gdn::ChunkArgs A{};
    A.x = x; A.x_stride = x_stride; A.a = a; A.b = b; A.ab_stride = ab_stride; A.n_rows = batch->n_rows;
    A.cu = batch->cu_seqlens; A.page_idx = batch->page_idx; A.has_init = batch->has_init; A.n_seqs = batch->n_seqs;
    A.conv_w = params->conv_w; A.a_log = params->a_log; A.dt_bias = params->dt_bias;
    A.conv_base = conv.base; A.conv_page_stride = conv.page_stride; A.conv_n_pages = conv.n_pages; A.sync = conv.sync;
    A.state = state.base; A.state_page_stride = state.page_stride; A.state_n_pages = state.n_pages;
    A.o = o; A.err = err; A.h_k = dims->h_k; A.h_v = dims->h_v; A.d_v = dims->d_v;
    A.scale = dims->scale; A.eps = dims->l2_eps;
    A.workspace = workspace;
    const int64_t max_len = batch->max_seqlen > 0 ? batch->max_seqlen : batch->n_rows;
    if (max_len > INT32_MAX) return GDN_ERR_ARG;
    return from_hip(gdn::launch_chunked(A, dims->d_k, dims->act_dtype, dims->state_dtype, (int)max_len,
                                        (hipStream_t)stream));
}

namespace {
// Kernel-time break-even of the two sequence paths on MI355X (uniform
// batches, d_k = d_v = 128, bf16 activations, fp32 state; the chunked form
// pays about 28 us for its two launches at any size): token by token is
// faster up to 32 rows per sequence for 1-2 sequences, up to 16 rows for 3-8
// (at 4 sequences and 32 rows the two are within 3%), and below 16 rows for
// more; the chunked form is faster everywhere past that.
constexpr int32_t kTokenMaxFew = 32;   // batches of 1-2 sequences
constexpr int32_t kTokenMaxMid = 16;   // 3-8 sequences
constexpr int32_t kTokenMaxMany = 8;   // larger batches
constexpr int32_t kPrefillChunk = 64;
}  // namespace

GDN_EXPORT int32_t gdn_prefill_path(const gdn_dims* dims, const gdn_batch* batch, int32_t token_max,
                                    int32_t* path) {
    int32_t st;
    if ((st = check_dims(dims)) != GDN_OK) return st;
    if ((st = check_batch(batch)) != GDN_OK) return st;
    if (!path) return GDN_ERR_ARG;
    const int64_t longest = batch->max_seqlen > 0 ? batch->max_seqlen : batch->n_rows;
    const int64_t limit = token_max >= 0     ? token_max
                          : batch->n_seqs <= 2 ? kTokenMaxFew
                          : batch->n_seqs <= 8 ? kTokenMaxMid
                                               : kTokenMaxMany;
    const bool chunked_ok = gdn::chunked_supported(dims->d_k, dims->d_v, kPrefillChunk);
    *path = (chunked_ok && longest > limit) ? GDN_PATH_CHUNKED : GDN_PATH_TOKEN;
    return GDN_OK;
}

GDN_EXPORT int32_t gdn_prefill(const gdn_dims* dims, const gdn_params* params, const void* x, int64_t x_stride,
                               const void* a, const void* b, int64_t ab_stride, const gdn_batch* batch,
                               gdn_conv_pool conv, gdn_state_pool state, float* o, int32_t token_max,
                               void* workspace, size_t ws_bytes, int32_t* path, int32_t* err, void* stream) {
    int32_t which = GDN_PATH_TOKEN;
    const int32_t st = gdn_prefill_path(dims, batch, token_max, &which);
    if (st != GDN_OK) return st;
    if (path) *path = which;
    if (which == GDN_PATH_CHUNKED)
        return gdn_chunked_prefill(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o, kPrefillChunk,
                                   workspace, ws_bytes, err, stream);
    return gdn_recurrent_seq(dims, params, x, x_stride, a, b, ab_stride, batch, conv, state, o, err, stream);
}

namespace {
// A prefix cache's pools: states of the state dtype, windows of W-1 rows.
int32_t check_prefix_cache(const gdn_dims* dims, const gdn_prefix_cache& c, bool need_index) {
    int32_t st;
    if (need_index && (!c.entry || !c.row)) return GDN_ERR_ARG;
    if ((st = check_state_pool(dims, c.state)) != GDN_OK) return st;
    if ((st = check_conv_pool(dims, c.conv, dims->conv_w - 1, false)) != GDN_OK) return st;
    return GDN_OK;
}
}  // namespace

GDN_EXPORT int32_t gdn_spec_verify_cached(const gdn_dims* dims, const gdn_params* params, int32_t layout,
                                          const void* x, int64_t x_stride, const void* a, const void* b,
                                          int64_t ab_stride, int32_t n_req, int32_t n_cand, const int32_t* req_page,
                                          const int32_t* num_accepted, const uint8_t* step_parity, void* pages,
                                          int64_t page_bytes, int32_t n_pages, gdn_conv_pool conv,
                                          const gdn_prefix_cache* cache, float* o, int32_t* err, void* stream) {
    int32_t st;
    if ((st = check_dims(dims)) != GDN_OK) return st;
    if ((st = check_params(params)) != GDN_OK) return st;
    gdn_spec_layout L{};
    if ((st = check_verify_call(dims, layout, x, x_stride, a, b, ab_stride, n_req, n_cand, req_page, num_accepted,
                                step_parity, pages, page_bytes, n_pages, conv, o, &L)) != GDN_OK)
        return st;
    if (cache && (st = check_prefix_cache(dims, *cache, true)) != GDN_OK) return st;
    if (n_req == 0) return GDN_OK;
    gdn::VerifyArgs A = verify_args(dims, params, L, x, x_stride, a, b, ab_stride, n_req, n_cand, req_page,
                                    num_accepted, step_parity, pages, page_bytes, n_pages, conv, o, err);
    if (cache) {
        A.cache_entry = cache->entry; A.cache_row = cache->row;
        A.cache_state = cache->state.base; A.cache_state_stride = cache->state.page_stride;
        A.cache_state_n = cache->state.n_pages;
        A.cache_conv = cache->conv.base; A.cache_conv_stride = cache->conv.page_stride;
        A.cache_conv_n = cache->conv.n_pages;
    }
    return from_hip(gdn::launch_verify(A, dims->d_k, dims->act_dtype, dims->state_dtype, layout,
                                       (hipStream_t)stream));
}

GDN_EXPORT int32_t gdn_spec_verify(const gdn_dims* dims, const gdn_params* params, int32_t layout, const void* x,
                                   int64_t x_stride, const void* a, const void* b, int64_t ab_stride, int32_t n_req,
                                   int32_t n_cand, const int32_t* req_page, const int32_t* num_accepted,
                                   const uint8_t* step_parity, void* pages, int64_t page_bytes, int32_t n_pages,
                                   gdn_conv_pool conv, float* o, int32_t* err, void* stream) {
    return gdn_spec_verify_cached(dims, params, layout, x, x_stride, a, b, ab_stride, n_req, n_cand, req_page,
                                  num_accepted, step_parity, pages, page_bytes, n_pages, conv, nullptr, o, err,
                                  stream);
}

GDN_EXPORT int32_t gdn_prefix_restore(const gdn_dims* dims, int32_t layout, int32_t n_req, const int32_t* entry,
                                      const int32_t* req_page, const gdn_prefix_cache* cache, void* pages,
                                      int64_t page_bytes, int32_t n_pages, gdn_conv_pool conv, int32_t* err,
                                      void* stream) {
    int32_t st;
    if ((st = check_dims(dims)) != GDN_OK) return st;
    gdn_spec_layout L{};
    if ((st = gdn_spec_page_layout(dims, layout, &L)) != GDN_OK) return st;
    if (n_req < 0 || !cache) return GDN_ERR_ARG;
    if (n_req == 0) return GDN_OK;
    if (!entry || !req_page || !pages || n_pages < 0) return GDN_ERR_ARG;
    if (page_bytes < (int64_t)L.page_bytes || page_bytes % 256 != 0 || !aligned(pages, 256)) return GDN_ERR_ARG;
    if ((st = check_conv_pool(dims, conv, dims->conv_w - 1, false)) != GDN_OK) return st;
    if ((st = check_prefix_cache(dims, *cache, false)) != GDN_OK) return st;
    gdn::RestoreArgs A{};
    A.n_req = n_req; A.entry = entry; A.req_page = req_page;
    A.cache_state = cache->state.base; A.cache_state_stride = cache->state.page_stride;
    A.cache_state_n = cache->state.n_pages;
    A.cache_conv = cache->conv.base; A.cache_conv_stride = cache->conv.page_stride; A.cache_conv_n = cache->conv.n_pages;
    A.pages = static_cast<uint8_t*>(pages); A.page_bytes = page_bytes; A.n_pages = n_pages;
    A.header_off = (int64_t)L.header_off; A.state_off = (int64_t)L.state_off;
    A.conv_base = conv.base; A.conv_page_stride = conv.page_stride; A.conv_n_pages = conv.n_pages;
    A.err = err; A.h_v = dims->h_v; A.d_k = dims->d_k; A.d_v = dims->d_v; A.conv_rows = dims->conv_w - 1;
    A.C = (int32_t)c_conv(dims);
    return from_hip(gdn::launch_restore(A, dims->act_dtype, dims->state_dtype, (hipStream_t)stream));
}

namespace {
bool mixed_two_launches(const gdn_dims* dims, const gdn_seq_part* seq, const gdn_verify_part* verify) {
    return seq && verify && seq->batch && seq->batch->n_seqs > 0 && verify->n_req > 0 && !seq->spec_pages &&
           seq->batch->max_seqlen >= 1 && seq->batch->max_seqlen <= 4 && dims->d_v % 64 == 0;
}
}  // namespace

GDN_EXPORT int32_t gdn_mixed_launches(const gdn_dims* dims, const gdn_seq_part* seq, const gdn_verify_part* verify,
                                      int32_t* launches) {
    int32_t st;
    if ((st = check_dims(dims)) != GDN_OK) return st;
    if (!launches) return GDN_ERR_ARG;
    if (seq && (st = check_batch(seq->batch)) != GDN_OK) return st;
    *launches = mixed_two_launches(dims, seq, verify) ? GDN_MIXED_TWO_LAUNCHES : GDN_MIXED_ONE_LAUNCH;
    return GDN_OK;
}

GDN_EXPORT int32_t gdn_mixed_step_launches(const gdn_dims* dims, const gdn_params* params, const gdn_seq_part* seq,
                                           const gdn_verify_part* verify, int32_t launches, int32_t* err,
                                           void* stream) {
    int32_t st;
    if ((st = check_dims(dims)) != GDN_OK) return st;
    if ((st = check_params(params)) != GDN_OK) return st;
    if (launches != GDN_MIXED_AUTO && launches != GDN_MIXED_ONE_LAUNCH && launches != GDN_MIXED_TWO_LAUNCHES)
        return GDN_ERR_ARG;
    gdn::SeqArgs S{};
    gdn::VerifyArgs V{};
    int32_t layout = GDN_SPEC_ONEPAGE;
    if (seq) {
        if ((st = check_sequence_call(dims, params, seq->x, seq->x_stride, seq->a, seq->b, seq->ab_stride,
                                      seq->batch, seq->conv, seq->state, seq->o)) != GDN_OK)
            return st;
        if (seq->spec_pages && (seq->spec_page_bytes < 256 || seq->spec_page_bytes % 256 != 0 ||
                                !aligned(seq->spec_pages, 256) || seq->spec_n_pages < 0))
            return GDN_ERR_ARG;
        if (seq->batch->n_seqs > 0) {
            S = seq_args(dims, params, seq->x, seq->x_stride, seq->a, seq->b, seq->ab_stride, seq->batch, seq->conv,
                         seq->state, seq->o, err);
            S.spec_pages = static_cast<uint8_t*>(seq->spec_pages);
            S.spec_page_bytes = seq->spec_page_bytes;
            S.spec_n_pages = seq->spec_n_pages;
        }
    }
    if (verify) {
        gdn_spec_layout L{};
        const gdn_verify_part& v = *verify;
        if ((st = check_verify_call(dims, v.layout, v.x, v.x_stride, v.a, v.b, v.ab_stride, v.n_req, v.n_cand,
                                    v.req_page, v.num_accepted, v.step_parity, v.pages, v.page_bytes, v.n_pages,
                                    v.conv, v.o, &L)) != GDN_OK)
            return st;
        layout = v.layout;
        if (v.n_req > 0)
            V = verify_args(dims, params, L, v.x, v.x_stride, v.a, v.b, v.ab_stride, v.n_req, v.n_cand, v.req_page,
                            v.num_accepted, v.step_parity, v.pages, v.page_bytes, v.n_pages, v.conv, v.o, err);
    }
    if (S.n_seqs == 0 && V.n_req == 0) return GDN_OK;
    const bool two = launches == GDN_MIXED_TWO_LAUNCHES ||
                     (launches == GDN_MIXED_AUTO && mixed_two_launches(dims, seq, verify));
    if (two) {
        // the sequences first, on gdn_recurrent_seq's kernel for their shape (its
        // 32-column kernel when they also write speculative-page headers, which
        // the short-sequence kernel does not do), then the verify requests
        if (S.n_seqs > 0) {
            const int max_len = S.spec_pages ? 0 : seq->batch->max_seqlen;
            if ((st = from_hip(gdn::launch_seq(S, dims->d_k, dims->act_dtype, dims->state_dtype, max_len,
                                               (hipStream_t)stream))) != GDN_OK)
                return st;
        }
        if (V.n_req > 0)
            return from_hip(gdn::launch_verify(V, dims->d_k, dims->act_dtype, dims->state_dtype, layout,
                                               (hipStream_t)stream));
        return GDN_OK;
    }
    return from_hip(gdn::launch_mixed(S, V, dims->d_k, dims->act_dtype, dims->state_dtype, layout,
                                      (hipStream_t)stream));
}

GDN_EXPORT int32_t gdn_mixed_step(const gdn_dims* dims, const gdn_params* params, const gdn_seq_part* seq,
                                  const gdn_verify_part* verify, int32_t* err, void* stream) {
    return gdn_mixed_step_launches(dims, params, seq, verify, GDN_MIXED_AUTO, err, stream);
}
