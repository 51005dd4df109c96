// C ABI of libpkd: argument validation, typed refusals with numbers, pool
// layout, workspace carving and the decode-step composition.  Allocates no
// device memory; every launch is asynchronous on the caller's stream.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"

namespace pkd {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

pkd_status fail(pkd_error* err, pkd_status code, int64_t needed, int64_t available, const char* fmt, ...) {
  if (err) {
    err->code = code;
    err->needed = needed;
    err->available = available;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(err->detail, sizeof(err->detail), fmt, ap);
    va_end(ap);
  }
  return code;
}

pkd_status ok(pkd_error* err) {
  if (err) {
    err->code = PKD_OK;
    err->needed = 0;
    err->available = 0;
    err->detail[0] = 0;
  }
  return PKD_OK;
}

pkd_status check_launch(pkd_error* err, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(err, PKD_ERR_DEVICE, 0, 0, "%s: %s", what, hipGetErrorString(e));
  return ok(err);
}

int elem_size(int dtype) { return dtype == PKD_F32 ? 4 : dtype == PKD_BF16 ? 2 : 1; }

static bool valid_dtype(int d) { return d == PKD_F32 || d == PKD_BF16 || d == PKD_FP8_E4M3; }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Layout of a pool; returns false for an invalid descriptor.
static bool pool_layout(const pkd_pool_desc* d, pkd_pool_info* info) {
  if (!d || d->num_pages < 1 || d->page_tokens != kPage || d->num_kv_heads < 1 ||
      (d->head_dim != 64 && d->head_dim != 128) || !valid_dtype(d->kv_dtype) || d->max_seqs < 1 ||
      d->max_pages_per_seq < 1 || d->attn_chunk_pages < 1)
    return false;
  const size_t block = (size_t)kPage * d->head_dim * elem_size(d->kv_dtype);
  pkd_pool_info in{};
  in.pages_offset = 0;
  in.block_bytes = block;
  size_t off = align256((size_t)d->num_pages * d->num_kv_heads * 2 * block);
  in.table_offset = off;
  off += align256(sizeof(int32_t) * (size_t)d->max_seqs * d->max_pages_per_seq);
  in.counts_offset = off;
  off += align256(sizeof(int32_t) * (size_t)d->max_seqs);
  in.error_offset = off;
  off += 256;
  in.total_bytes = off;
  if (info) *info = in;
  return true;
}

// Fill of int32 words on the stream (a kernel, so that the call can sit in a
// captured graph).
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void cast_bf16_kernel(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; 4 * i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(x + 4 * i);
    *reinterpret_cast<u32x2*>(y + 4 * i) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
}

pkd_status cast_bf16_launch(const float* x, void* y, int64_t n, hipStream_t stream, pkd_error* err) {
  if (n <= 0) return ok(err);
  const int64_t blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, x,
                     (uint16_t*)y, n);
  return check_launch(err, "cast to bf16");
}

static pkd_status validate_pool(const pkd_pool* pool, pkd_error* err) {
  if (!pool || !pool->base) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "pool is NULL");
  return PKD_OK;
}

static pkd_status validate_rows(const pkd_rows* rows, pkd_error* err) {
  if (!rows) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "rows is NULL");
  if (rows->n < 0) return fail(err, PKD_ERR_INVALID_ARG, rows->n, 0, "negative row count %d", rows->n);
  if (rows->n > 0 && (!rows->seq || !rows->pos))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "rows->seq / rows->pos is NULL");
  if (rows->flags & ~PKD_ROWS_DISTINCT_SEQS)
    return fail(err, PKD_ERR_INVALID_ARG, rows->flags, PKD_ROWS_DISTINCT_SEQS, "unknown rows->flags bits");
  return PKD_OK;
}

pkd_status proj_validate(const ProjArgs& a, pkd_error* err) {
  const pkd_matrix* W = a.W;
  if (!W || !W->data) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "matrix or its data is NULL");
  if (!valid_dtype(W->dtype)) return fail(err, PKD_ERR_INVALID_ARG, W->dtype, 0, "bad weight dtype %d", W->dtype);
  if (W->family != PKD_FAMILY_GEMV && W->family != PKD_FAMILY_MFMA && W->family != PKD_FAMILY_MFMA_FP8 &&
      W->family != PKD_FAMILY_GEMV_MFMA)
    return fail(err, PKD_ERR_INVALID_ARG, W->family, 0, "bad family %d", W->family);
  if (W->family == PKD_FAMILY_MFMA_FP8 && W->dtype != PKD_FP8_E4M3)
    return fail(err, PKD_ERR_UNSUPPORTED, W->dtype, PKD_FP8_E4M3, "the native fp8 family needs fp8 weights");
  if (W->rows < 1 || W->cols < 64 || W->cols % 64)
    return fail(err, PKD_ERR_UNSUPPORTED, W->cols, 64, "matrix %d x %d: cols must be a positive multiple of 64",
                W->rows, W->cols);
  if (!(W->scale > 0.f) || !isfinite(W->scale))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "weight scale must be finite and positive");
  if (W->dtype != PKD_FP8_E4M3 && W->scale != 1.0f)
    return fail(err, PKD_ERR_UNSUPPORTED, 0, 0, "a per-tensor scale is only supported for fp8 weights");
  if (a.n_rows < 0) return fail(err, PKD_ERR_INVALID_ARG, a.n_rows, 0, "negative row count");
  if (a.x_dtype != PKD_F32 && a.x_dtype != PKD_BF16)
    return fail(err, PKD_ERR_UNSUPPORTED, a.x_dtype, 0, "activations must be f32 or bf16");
  if (a.out_dtype != PKD_F32 && a.out_dtype != PKD_BF16)
    return fail(err, PKD_ERR_UNSUPPORTED, a.out_dtype, 0, "output must be f32 or bf16");
  if (a.silu_pair && (W->rows % 2 || a.residual))
    return fail(err, PKD_ERR_INVALID_ARG, W->rows, 0, "silu_pair needs an even row count and no residual");
  if (a.n_rows > 0 && (!a.x || !a.y)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "x or y is NULL");
  if (a.rope_cs) {
    const int n_out = a.silu_pair ? W->rows / 2 : W->rows;
    if (a.silu_pair) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "rotary pairs and silu_pair exclude each other");
    if (a.rope_hd < 4 || a.rope_hd % 4 || a.rope_cols < 0 || a.rope_cols % a.rope_hd || a.rope_cols > n_out)
      return fail(err, PKD_ERR_INVALID_ARG, a.rope_cols, n_out,
                  "rope_head_dim %d must be a positive multiple of 4 and rope_cols %d a multiple of it, at most %d",
                  a.rope_hd, a.rope_cols, n_out);
  }
  if (((uintptr_t)a.row_scale & 3) || ((uintptr_t)a.rope_cs & 7))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "row_scale must be 4-byte and rope_cs 8-byte aligned");
  if (!aligned16(a.x) || !aligned16(a.y) || !aligned16(a.residual) || !aligned16(a.y_bf16))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "device pointers must be 16-byte aligned");
  if (W->family == PKD_FAMILY_GEMV_MFMA) {
    if (W->dtype == PKD_F32 || a.x_dtype != PKD_BF16)
      return fail(err, PKD_ERR_UNSUPPORTED, a.x_dtype, PKD_BF16,
                  "the GEMV_MFMA family needs bf16 or fp8 weights and bf16 activations");
  }
  if (tiled_family(W->family)) {
    const int kb = W->family == PKD_FAMILY_MFMA_FP8 ? 128 : 64;
    if (W->dtype == PKD_F32) return fail(err, PKD_ERR_UNSUPPORTED, 0, 0, "matrix-core family needs bf16 or fp8 weights");
    if (W->rows % 128 || W->cols % kb)
      return fail(err, PKD_ERR_UNSUPPORTED, W->rows, 128,
                  "matrix-core family needs rows %% 128 == 0 and cols %% %d == 0 (got %d x %d)", kb, W->rows, W->cols);
    if (W->dtype == PKD_BF16 && a.x_dtype != PKD_BF16)
      return fail(err, PKD_ERR_UNSUPPORTED, a.x_dtype, PKD_BF16, "bf16 matrix-core family needs bf16 activations");
    if (W->k_splits < 0 || W->k_splits > W->cols / kb)
      return fail(err, PKD_ERR_UNSUPPORTED, W->k_splits, W->cols / kb, "k_splits %d outside 0..%d for %d columns",
                  W->k_splits, W->cols / kb, W->cols);
  }
  return PKD_OK;
}

}  // namespace pkd

using namespace pkd;

extern "C" {

const char* pkd_version(void) { return "pkd 0.1 (gfx950)"; }

const char* pkd_status_string(int32_t s) {
  switch (s) {
    case PKD_OK: return "ok";
    case PKD_ERR_INVALID_ARG: return "invalid argument";
    case PKD_ERR_UNSUPPORTED: return "unsupported";
    case PKD_ERR_OUT_OF_MEMORY: return "out of memory";
    case PKD_ERR_BOUNDS: return "out of bounds";
    case PKD_ERR_DUPLICATE_PAGE: return "duplicate page";
    case PKD_ERR_DEVICE: return "device error";
    case PKD_ERR_ROW: return "invalid row";
    default: return "unknown status";
  }
}

size_t pkd_pool_bytes(const pkd_pool_desc* desc) {
  pkd_pool_info info;
  if (!pool_layout(desc, &info)) return 0;
  return info.total_bytes;
}

pkd_status kv_pool_create(const pkd_pool_desc* desc, void* dev_mem, size_t bytes, pkd_stream stream,
                          pkd_pool** out, pkd_error* err) {
  if (!desc || !out) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "desc or out is NULL");
  *out = nullptr;
  if (desc->page_tokens != kPage)
    return fail(err, PKD_ERR_UNSUPPORTED, desc->page_tokens, kPage, "page_tokens must be 32");
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(err, PKD_ERR_UNSUPPORTED, desc->head_dim, 128, "head_dim must be 64 or 128");
  if (!valid_dtype(desc->kv_dtype)) return fail(err, PKD_ERR_INVALID_ARG, desc->kv_dtype, 0, "bad kv dtype");
  if (desc->kv_dtype == PKD_FP8_E4M3) {
    if (!(desc->k_scale > 0.f) || !(desc->v_scale > 0.f) || !isfinite(desc->k_scale) || !isfinite(desc->v_scale))
      return fail(err, PKD_ERR_UNSUPPORTED, 0, 0, "fp8 scales must be finite and positive");
  } else if (desc->k_scale != 1.0f || desc->v_scale != 1.0f) {
    return fail(err, PKD_ERR_UNSUPPORTED, 0, 0, "k_scale and v_scale must be 1 for a non-fp8 pool");
  }
  pkd_pool_info info;
  if (!pool_layout(desc, &info))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "invalid pool descriptor (counts must be >= 1)");
  if (!dev_mem) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "dev_mem is NULL");
  if ((uintptr_t)dev_mem & 255) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "dev_mem must be 256-byte aligned");
  if (bytes < info.total_bytes)
    return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)info.total_bytes, (int64_t)bytes,
                "pool needs %zu bytes, buffer has %zu", info.total_bytes, bytes);
  pkd_pool* p = (pkd_pool*)calloc(1, sizeof(pkd_pool));
  if (!p) return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)sizeof(pkd_pool), 0, "host allocation of the handle failed");
  const int64_t tab = (int64_t)desc->max_seqs * desc->max_pages_per_seq;
  p->page_refs = (int32_t*)calloc((size_t)desc->num_pages, sizeof(int32_t));
  p->host_table = (int32_t*)malloc(sizeof(int32_t) * (size_t)tab);
  p->host_counts = (int32_t*)calloc((size_t)desc->max_seqs, sizeof(int32_t));
  if (!p->page_refs || !p->host_table || !p->host_counts) {
    free(p->page_refs);
    free(p->host_table);
    free(p->host_counts);
    free(p);
    return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)desc->num_pages * 4 + tab * 4, 0,
                "host allocation of the pool's table copy failed");
  }
  for (int64_t i = 0; i < tab; ++i) p->host_table[i] = -1;
  p->desc = *desc;
  p->base = (uint8_t*)dev_mem;
  p->bytes = bytes;
  p->info = info;
  (void)hipGetDevice(&p->device);
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(256), dim3(256), 0, st, (int32_t*)(p->base + info.table_offset), tab, -1);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(64), dim3(256), 0, st, (int32_t*)(p->base + info.counts_offset),
                     (int64_t)desc->max_seqs, 0);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, (int32_t*)(p->base + info.error_offset), 64, 0);
  pkd_status s = check_launch(err, "kv_pool_create");
  // the fills land before the call returns, so that a later call on any
  // stream (block_table_set included) sees the laid-out pool
  if (s == PKD_OK) {
    const hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) s = fail(err, PKD_ERR_DEVICE, 0, 0, "kv_pool_create: %s", hipGetErrorString(e));
  }
  if (s != PKD_OK) {
    free(p->page_refs);
    free(p->host_table);
    free(p->host_counts);
    free(p);
    return s;
  }
  *out = p;
  return ok(err);
}

pkd_status kv_pool_destroy(pkd_pool* pool) {
  if (pool) {
    free(pool->page_refs);
    free(pool->host_table);
    free(pool->host_counts);
  }
  free(pool);
  return PKD_OK;
}

pkd_status pkd_pool_info_get(const pkd_pool* pool, pkd_pool_info* info) {
  if (!pool || !info) return PKD_ERR_INVALID_ARG;
  *info = pool->info;
  info->shared_pages = pool->shared_pages;
  return PKD_OK;
}

pkd_status block_table_set(pkd_pool* pool, int32_t first_seq, int32_t n_seqs, const int32_t* pages_host,
                           const int32_t* n_pages_host, pkd_stream stream, pkd_error* err) {
  if (validate_pool(pool, err)) return PKD_ERR_INVALID_ARG;
  const pkd_pool_desc& d = pool->desc;
  if (n_seqs < 0 || first_seq < 0 || (n_seqs > 0 && (!pages_host || !n_pages_host)))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "bad sequence range or NULL host arrays");
  if ((int64_t)first_seq + n_seqs > d.max_seqs)
    return fail(err, PKD_ERR_BOUNDS, (int64_t)first_seq + n_seqs, d.max_seqs,
                "sequences %d..%d past max_seqs %d", first_seq, first_seq + n_seqs - 1, d.max_seqs);
  if (n_seqs == 0) return ok(err);
  const int mp = d.max_pages_per_seq;
  std::vector<int32_t> table((size_t)n_seqs * mp, -1);
  std::vector<uint32_t> seen((size_t)d.num_pages, 0);  // stamp = sequence index + 1
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t n = n_pages_host[i];
    if (n < 0 || n > mp)
      return fail(err, PKD_ERR_BOUNDS, n, mp, "sequence %d asks for %d pages, at most %d per sequence",
                  first_seq + i, n, mp);
    for (int32_t j = 0; j < n; ++j) {
      const int32_t pg = pages_host[(size_t)i * mp + j];
      if (pg < 0 || pg >= d.num_pages)
        return fail(err, PKD_ERR_BOUNDS, pg, d.num_pages, "sequence %d page %d: id %d outside the pool of %d pages",
                    first_seq + i, j, pg, d.num_pages);
      if (seen[pg] == (uint32_t)i + 1)
        return fail(err, PKD_ERR_DUPLICATE_PAGE, pg, 0, "sequence %d lists page %d twice", first_seq + i, pg);
      seen[pg] = (uint32_t)i + 1;
      table[(size_t)i * mp + j] = pg;
    }
  }
  hipStream_t st = (hipStream_t)stream;
  int32_t* dt = (int32_t*)(pool->base + pool->info.table_offset) + (size_t)first_seq * mp;
  int32_t* dc = (int32_t*)(pool->base + pool->info.counts_offset) + first_seq;
  // The tables being replaced come from the handle's host copy (no read-back),
  // which keeps the per-page sequence counts exact.
  int32_t* ht = pool->host_table + (size_t)first_seq * mp;
  int32_t* hc = pool->host_counts + first_seq;
  for (int32_t i = 0; i < n_seqs; ++i) {
    for (int32_t j = 0; j < hc[i]; ++j) {
      const int32_t pg = ht[(size_t)i * mp + j];
      if (pool->page_refs[pg] > 0 && --pool->page_refs[pg] == 1) --pool->shared_pages;
    }
    for (int32_t j = 0; j < n_pages_host[i]; ++j)
      if (++pool->page_refs[table[(size_t)i * mp + j]] == 2) ++pool->shared_pages;
    hc[i] = n_pages_host[i];
  }
  memcpy(ht, table.data(), sizeof(int32_t) * table.size());
  hipError_t e = hipMemcpyAsync(dt, ht, sizeof(int32_t) * table.size(), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(dc, hc, sizeof(int32_t) * (size_t)n_seqs, hipMemcpyHostToDevice, st);
  // returns once the tables are on the device (the host copy may change with
  // the next call)
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(err, PKD_ERR_DEVICE, 0, 0, "block_table_set: %s", hipGetErrorString(e));
  return ok(err);
}

pkd_status pkd_pool_check(pkd_pool* pool, pkd_stream stream, pkd_error* err) {
  if (validate_pool(pool, err)) return PKD_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  uint32_t word = 0;
  uint32_t* dev = (uint32_t*)(pool->base + pool->info.error_offset);
  hipError_t e = hipMemcpyAsync(&word, dev, sizeof(word), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && word) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, (int32_t*)dev, 1, 0);
    e = hipStreamSynchronize(st);
  }
  if (e != hipSuccess) return fail(err, PKD_ERR_DEVICE, 0, 0, "pkd_pool_check: %s", hipGetErrorString(e));
  if (word)
    return fail(err, PKD_ERR_ROW, word, 0, "invalid rows were zero-filled (bits %u: 1 seq, 2 pos, 4 page)", word);
  return ok(err);
}

size_t pkd_attn_workspace_bytes(const pkd_pool* pool, int32_t n_q_heads, int32_t max_rows) {
  return attn_workspace_bytes(pool, n_q_heads, max_rows);
}

static pkd_status validate_attn(pkd_pool* pool, const pkd_rows* rows, int32_t n_q_heads, const void* q,
                                const void* k_new, const void* v_new, void* out, int32_t out_dtype, pkd_error* err) {
  if (validate_pool(pool, err) || validate_rows(rows, err)) return err ? (pkd_status)err->code : PKD_ERR_INVALID_ARG;
  const int kv = pool->desc.num_kv_heads;
  if (n_q_heads < kv || n_q_heads % kv || n_q_heads / kv > 16)
    return fail(err, PKD_ERR_UNSUPPORTED, n_q_heads, kv,
                "n_q_heads %d must be G x num_kv_heads (%d) with 1 <= G <= 16", n_q_heads, kv);
  if (out_dtype != PKD_F32 && out_dtype != PKD_BF16)
    return fail(err, PKD_ERR_UNSUPPORTED, out_dtype, 0, "attention output must be f32 or bf16");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "k_new and v_new must both be given or both be NULL");
  if (rows->n > 0 && (!q || !out)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "q or out is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_new) || !aligned16(v_new))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "device pointers must be 16-byte aligned");
  return PKD_OK;
}

pkd_status paged_attn_decode(pkd_pool* pool, const pkd_rows* rows, int32_t n_q_heads, const void* q,
                             const void* k_new, const void* v_new, void* out, int32_t out_dtype, void* ws,
                             size_t ws_bytes, pkd_stream stream, pkd_error* err) {
  pkd_status s = validate_attn(pool, rows, n_q_heads, q, k_new, v_new, out, out_dtype, err);
  if (s != PKD_OK) return s;
  const int d = pool->desc.head_dim;
  AttnArgs a{};
  a.pool = pool;
  a.seq = rows->seq;
  a.pos = rows->pos;
  a.distinct = (rows->flags & PKD_ROWS_DISTINCT_SEQS) != 0;
  a.n_rows = rows->n;
  a.n_q_heads = n_q_heads;
  a.q = q;
  a.q_stride = (int64_t)n_q_heads * d;
  a.k_new = k_new;
  a.v_new = v_new;
  a.kv_new_stride = (int64_t)pool->desc.num_kv_heads * d;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_stride = (int64_t)n_q_heads * d;
  return attn_launch(a, ws, ws_bytes, (hipStream_t)stream, err);
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation attention
// Scratch of paged_attn_decode_noalloc: the chunk records of chunked pools,
// in a fixed device array that every GPU the library runs on holds for the
// life of the process.  Host code never uses the array's name as an address:
// its device address is looked up once per device (with that device current)
// and kept in scratch_dev.
namespace pkd {
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
}  // namespace pkd
static __device__ __align__(256) uint8_t scratch[pkd::kNoAllocScratchBytes];
static void* scratch_dev[pkd::kMaxDevices];
static std::mutex scratch_mu;

static pkd_status scratch_address(void** out, pkd_error* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(err, PKD_ERR_DEVICE, 0, 0, "paged_attn_decode_noalloc: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(err, PKD_ERR_UNSUPPORTED, dev, kMaxDevices, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(err, PKD_ERR_DEVICE, 0, 0, "paged_attn_decode_noalloc: scratch address: %s", hipGetErrorString(e));
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return PKD_OK;
}

extern "C" {

size_t pkd_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

pkd_status paged_attn_decode_noalloc(pkd_pool* pool, const pkd_rows* rows, int32_t n_q_heads, const void* q,
                                     const void* k_new, const void* v_new, void* out, int32_t out_dtype,
                                     pkd_stream stream, pkd_error* err) {
  pkd_status s = validate_attn(pool, rows, n_q_heads, q, k_new, v_new, out, out_dtype, err);
  if (s != PKD_OK) return s;
  const size_t need = attn_workspace_bytes(pool, n_q_heads, rows->n);
  if (need > kNoAllocScratchBytes)
    return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)need, (int64_t)kNoAllocScratchBytes,
                "paged_attn_decode_noalloc: %d rows need %zu bytes of chunk records, more than its fixed "
                "%zu-byte scratch; use paged_attn_decode with a workspace",
                rows->n, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0 && (s = scratch_address(&ws, err)) != PKD_OK) return s;
  const int d = pool->desc.head_dim;
  AttnArgs a{};
  a.pool = pool;
  a.seq = rows->seq;
  a.pos = rows->pos;
  a.distinct = (rows->flags & PKD_ROWS_DISTINCT_SEQS) != 0;
  a.n_rows = rows->n;
  a.n_q_heads = n_q_heads;
  a.q = q;
  a.q_stride = (int64_t)n_q_heads * d;
  a.k_new = k_new;
  a.v_new = v_new;
  a.kv_new_stride = (int64_t)pool->desc.num_kv_heads * d;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_stride = (int64_t)n_q_heads * d;
  return attn_launch(a, ws, need > 0 ? kNoAllocScratchBytes : 0, (hipStream_t)stream, err);
}

size_t pkd_gemv_workspace_bytes(const pkd_matrix* W, int32_t max_rows) { return proj_workspace_bytes(W, max_rows); }

int32_t pkd_suggest_k_splits(int32_t rows, int32_t cols, int32_t family, int32_t typical_rows) {
  return suggest_k_splits(rows, cols, family, typical_rows);
}

pkd_status gemv_rows(const pkd_matrix* W, const void* x, int32_t x_dtype, int32_t n_rows, void* y,
                     const pkd_epilogue* ep, void* ws, size_t ws_bytes, pkd_stream stream, pkd_error* err) {
  if (!ep) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "epilogue is NULL");
  ProjArgs a{};
  a.W = W;
  a.x = x;
  a.x_dtype = x_dtype;
  a.n_rows = n_rows;
  a.y = y;
  a.out_dtype = ep->out_dtype;
  a.residual = ep->residual;
  a.silu_pair = ep->silu_pair;
  a.y_bf16 = ep->y_bf16;
  a.row_scale = ep->row_scale;
  a.rope_cs = ep->rope_cs;
  a.rope_cols = ep->rope_cols;
  a.rope_hd = ep->rope_head_dim;
  pkd_status s = proj_validate(a, err);
  if (s != PKD_OK) return s;
  return proj_launch(a, ws, ws_bytes, (hipStream_t)stream, err);
}

pkd_status gemv_gather_rows(const pkd_matrix* W, const void* x, int32_t x_dtype, int32_t n_rows,
                            const int32_t* cand, const int32_t* n_cand, int32_t max_cand, float* y,
                            pkd_stream stream, pkd_error* err) {
  ProjArgs a{};
  a.W = W;
  a.x = x;
  a.x_dtype = x_dtype;
  a.n_rows = n_rows;
  a.y = y;
  a.out_dtype = PKD_F32;
  pkd_status s = proj_validate(a, err);
  if (s != PKD_OK) return s;
  if (tiled_family(W->family))
    return fail(err, PKD_ERR_UNSUPPORTED, W->family, PKD_FAMILY_GEMV,
                "gathered rows are evaluated with the GEMV families' summation orders only");
  if (n_rows > 65535) return fail(err, PKD_ERR_UNSUPPORTED, n_rows, 65535, "at most 65535 activation rows");
  if (n_rows == 0) return PKD_OK;
  if (max_cand < 1) return fail(err, PKD_ERR_INVALID_ARG, max_cand, 1, "max_cand must be positive");
  if (!cand || !n_cand) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "cand or n_cand is NULL");
  if (((uintptr_t)cand | (uintptr_t)n_cand) & 3)
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "cand and n_cand must be 4-byte aligned");
  return gemv_gather_launch(*W, x, x_dtype, n_rows, cand, n_cand, max_cand, y, (hipStream_t)stream, err);
}

pkd_status rms_norm_factor(const float* x, int32_t n_rows, int32_t cols, float eps, float* inv_rms, void* x_bf16,
                           pkd_stream stream, pkd_error* err) {
  if (n_rows < 0) return fail(err, PKD_ERR_INVALID_ARG, n_rows, 0, "negative row count");
  if (cols < 4 || cols % 4) return fail(err, PKD_ERR_UNSUPPORTED, cols, 4, "cols must be a positive multiple of 4");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "eps must be finite and >= 0");
  if (n_rows == 0) return ok(err);
  if (!x || !inv_rms) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "x or inv_rms is NULL");
  if (!aligned16(x) || !aligned16(x_bf16) || ((uintptr_t)inv_rms & 3))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "x and x_bf16 must be 16-byte aligned, inv_rms 4-byte");
  return rms_factor_launch(x, n_rows, cols, eps, inv_rms, x_bf16, (hipStream_t)stream, err);
}

pkd_status rope_table(const int32_t* pos, int32_t n_rows, int32_t head_dim, float base, float* cs, pkd_stream stream,
                      pkd_error* err) {
  if (n_rows < 0) return fail(err, PKD_ERR_INVALID_ARG, n_rows, 0, "negative row count");
  if (head_dim < 2 || head_dim % 2) return fail(err, PKD_ERR_INVALID_ARG, head_dim, 2, "head_dim must be even");
  if (!(base > 0.f) || !isfinite(base)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "base must be finite and > 0");
  if (n_rows == 0) return ok(err);
  if (!pos || !cs) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "pos or cs is NULL");
  if (((uintptr_t)pos & 3) || ((uintptr_t)cs & 7))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "pos must be 4-byte and cs 8-byte aligned");
  return rope_table_launch(pos, n_rows, head_dim, base, cs, (hipStream_t)stream, err);
}

// ------------------------------------------------------------------ decode step
struct StepWs {
  void* x_in;   // [n][D] bf16 (bf16 tier)
  void* qkv;    // [n][(Hq + 2Hkv) d] act
  void* attn;   // [n][Hq d] act
  float* h;     // [n][D] f32
  void* h_in;   // [n][D] bf16 (bf16 tier)
  void* a;      // [n][F] act
  void* attn_ws;
  size_t attn_ws_bytes;
  void* proj_ws;
  size_t proj_ws_bytes;
  float* inv_x;  // [n] norm factor of x (PKD_LAYER_NORM)
  float* inv_h;  // [n] norm factor of h
  float* cs;     // [n][d / 2][2] rotary table (PKD_LAYER_ROPE)
};

static size_t step_carve(const pkd_layer* L, const pkd_pool* pool, int32_t n, uint8_t* base, StepWs* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* p = base ? (void*)(base + off) : nullptr;
    off += align256(bytes);
    return p;
  };
  const int es = elem_size(L->act_dtype);
  const int nqkv = (L->n_q_heads + 2 * L->n_kv_heads) * L->head_dim;
  StepWs t{};
  const bool bf = L->act_dtype == PKD_BF16;
  t.x_in = bf ? take((size_t)n * L->hidden * 2) : nullptr;
  t.qkv = take((size_t)n * nqkv * es);
  t.attn = take((size_t)n * L->n_q_heads * L->head_dim * es);
  t.h = (float*)take((size_t)n * L->hidden * 4);
  t.h_in = bf ? take((size_t)n * L->hidden * 2) : nullptr;
  t.a = L->ffn > 0 ? take((size_t)n * L->ffn * es) : nullptr;
  t.attn_ws_bytes = attn_workspace_bytes(pool, L->n_q_heads, n);
  t.attn_ws = t.attn_ws_bytes ? take(t.attn_ws_bytes) : nullptr;
  size_t pw = proj_workspace_bytes(&L->w_qkv, n);
  pw = pw > proj_workspace_bytes(&L->w_o, n) ? pw : proj_workspace_bytes(&L->w_o, n);
  if (L->ffn > 0) {
    size_t g = proj_workspace_bytes(&L->w_gate_up, n), dn = proj_workspace_bytes(&L->w_down, n);
    pw = pw > g ? pw : g;
    pw = pw > dn ? pw : dn;
  }
  t.proj_ws_bytes = pw;
  t.proj_ws = pw ? take(pw) : nullptr;
  if (L->flags & PKD_LAYER_NORM) {
    t.inv_x = (float*)take((size_t)n * 4);
    t.inv_h = (float*)take((size_t)n * 4);
  }
  if (L->flags & PKD_LAYER_ROPE) t.cs = (float*)take((size_t)n * L->head_dim * 4);
  if (w) *w = t;
  return off;
}

size_t pkd_step_workspace_bytes(const pkd_layer* layer, const pkd_pool* pool, int32_t max_rows) {
  if (!layer || !pool || max_rows < 0) return 0;
  return step_carve(layer, pool, max_rows, nullptr, nullptr);
}

static pkd_status check_matrix(const pkd_matrix& W, int rows, int cols, const char* name, pkd_error* err) {
  if (W.rows != rows || W.cols != cols)
    return fail(err, PKD_ERR_INVALID_ARG, (int64_t)W.rows * 100000 + W.cols, (int64_t)rows * 100000 + cols,
                "%s is %d x %d, the layer needs %d x %d", name, W.rows, W.cols, rows, cols);
  return PKD_OK;
}

pkd_status decode_step(const pkd_layer* L, pkd_pool* pool, const pkd_rows* rows, const float* x, float* y, void* ws,
                       size_t ws_bytes, pkd_stream stream, pkd_error* err) {
  if (!L) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "layer is NULL");
  if (validate_pool(pool, err) || validate_rows(rows, err)) return err ? (pkd_status)err->code : PKD_ERR_INVALID_ARG;
  const pkd_pool_desc& pd = pool->desc;
  if (L->n_kv_heads != pd.num_kv_heads || L->head_dim != pd.head_dim)
    return fail(err, PKD_ERR_INVALID_ARG, L->n_kv_heads, pd.num_kv_heads, "layer kv heads / head_dim differ from the pool's");
  if (L->act_dtype != PKD_F32 && L->act_dtype != PKD_BF16)
    return fail(err, PKD_ERR_UNSUPPORTED, L->act_dtype, 0, "act_dtype must be f32 or bf16");
  if ((L->act_dtype == PKD_F32) != (pd.kv_dtype == PKD_F32))
    return fail(err, PKD_ERR_UNSUPPORTED, L->act_dtype, pd.kv_dtype, "an f32 layer needs an f32 pool and vice versa");
  if (L->hidden < 64 || L->hidden % 64 || L->ffn < 0 || L->ffn % 64)
    return fail(err, PKD_ERR_UNSUPPORTED, L->hidden, 64, "hidden and ffn must be multiples of 64");
  if (L->flags & ~(PKD_LAYER_NORM | PKD_LAYER_ROPE))
    return fail(err, PKD_ERR_INVALID_ARG, L->flags, PKD_LAYER_NORM | PKD_LAYER_ROPE, "unknown layer flags");
  if ((L->flags & PKD_LAYER_NORM) && (!(L->norm_eps >= 0.f) || !isfinite(L->norm_eps)))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "norm_eps must be finite and >= 0");
  if ((L->flags & PKD_LAYER_ROPE) && (!(L->rope_base > 0.f) || !isfinite(L->rope_base)))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "rope_base must be finite and > 0");
  const int D = L->hidden, d = L->head_dim, nq = L->n_q_heads, nkv = L->n_kv_heads, F = L->ffn;
  const int nqkv = (nq + 2 * nkv) * d;
  pkd_status s;
  if ((s = check_matrix(L->w_qkv, nqkv, D, "w_qkv", err))) return s;
  if ((s = check_matrix(L->w_o, D, nq * d, "w_o", err))) return s;
  if (F > 0) {
    if ((s = check_matrix(L->w_gate_up, 2 * F, D, "w_gate_up", err))) return s;
    if ((s = check_matrix(L->w_down, D, F, "w_down", err))) return s;
  }
  const int n = rows->n;
  if (n > 0 && (!x || !y)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "x and y must be 16-byte aligned");
  const size_t need = step_carve(L, pool, n, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)need, (int64_t)(ws ? ws_bytes : 0),
                "decode_step workspace needs %zu bytes", need);
  if ((uintptr_t)ws & 255) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "workspace must be 256-byte aligned");
  StepWs w;
  step_carve(L, pool, n, (uint8_t*)ws, &w);
  const bool bf = L->act_dtype == PKD_BF16;
  const int act = L->act_dtype;
  // projection inputs are taken in the activation dtype (the fp8 matrix-core
  // family quantises from the f32 / bf16 value itself)
  auto proj_in = [&](const pkd_matrix& W, const void* f32src, const void* bfsrc) -> std::pair<const void*, int> {
    if (!bf) return {f32src, PKD_F32};
    if (tiled_family(W.family) && W.dtype == PKD_FP8_E4M3 && f32src) return {f32src, PKD_F32};
    return {bfsrc, PKD_BF16};
  };
  ProjArgs p{};
  // validate all four projections before launching anything
  {
    ProjArgs v{};
    v.n_rows = n;
    v.x = ws;
    v.y = ws;
    v.out_dtype = act;
    v.W = &L->w_qkv;
    v.x_dtype = proj_in(L->w_qkv, x, w.x_in).second;
    if ((s = proj_validate(v, err))) return s;
    v.W = &L->w_o;
    v.x_dtype = act;
    v.out_dtype = PKD_F32;
    if ((s = proj_validate(v, err))) return s;
    if (F > 0) {
      v.W = &L->w_gate_up;
      v.x_dtype = proj_in(L->w_gate_up, w.h, w.h_in).second;
      v.out_dtype = act;
      v.silu_pair = 1;
      if ((s = proj_validate(v, err))) return s;
      v.W = &L->w_down;
      v.x_dtype = act;
      v.out_dtype = PKD_F32;
      v.silu_pair = 0;
      if ((s = proj_validate(v, err))) return s;
    }
  }
  hipStream_t st = (hipStream_t)stream;
  if (n == 0) return ok(err);
  // 1. qkv = W_qkv x  (norm: W_qkv carries the gain, outputs times 1/rms(x);
  //    rope: the q and k heads rotated by the row's position)
  const bool norm = (L->flags & PKD_LAYER_NORM) != 0, rope = (L->flags & PKD_LAYER_ROPE) != 0;
  // the vector GEMV rounds x to bf16 as it loads it, so that a decode batch
  // needs no pass of its own for the cast (the norm's pass writes the bf16 copy
  // anyway)
  const bool cast_in_gemv = bf && !norm && L->w_qkv.family == PKD_FAMILY_GEMV;
  const bool need_cast = bf && !(tiled_family(L->w_qkv.family) && L->w_qkv.dtype == PKD_FP8_E4M3) && !cast_in_gemv;
  if (norm) {
    if ((s = rms_factor_launch(x, n, D, L->norm_eps, w.inv_x, need_cast ? w.x_in : nullptr, st, err))) return s;
  } else if (need_cast && (s = cast_bf16_launch(x, w.x_in, (int64_t)n * D, st, err))) {
    return s;
  }
  if (rope && (s = rope_table_launch(rows->pos, n, d, L->rope_base, w.cs, st, err))) return s;
  const auto in0 = cast_in_gemv ? std::pair<const void*, int>{x, kXF32AsBf16} : proj_in(L->w_qkv, x, w.x_in);
  p = ProjArgs{};
  p.W = &L->w_qkv;
  p.x = in0.first;
  p.x_dtype = in0.second;
  p.n_rows = n;
  p.y = w.qkv;
  p.out_dtype = act;
  p.row_scale = norm ? w.inv_x : nullptr;
  p.rope_cs = rope ? w.cs : nullptr;
  p.rope_cols = (nq + nkv) * d;
  p.rope_hd = d;
  if ((s = proj_launch(p, w.proj_ws, w.proj_ws_bytes, st, err))) return s;
  // 2-3. append own k, v; attention over 0..pos
  AttnArgs a{};
  a.pool = pool;
  a.seq = rows->seq;
  a.pos = rows->pos;
  a.distinct = (rows->flags & PKD_ROWS_DISTINCT_SEQS) != 0;
  a.n_rows = n;
  a.n_q_heads = nq;
  const int es = elem_size(act);
  a.q = w.qkv;
  a.q_stride = nqkv;
  a.k_new = (const uint8_t*)w.qkv + (size_t)nq * d * es;
  a.v_new = (const uint8_t*)w.qkv + (size_t)(nq + nkv) * d * es;
  a.kv_new_stride = nqkv;
  a.out = w.attn;
  a.out_dtype = act;
  a.out_stride = (int64_t)nq * d;
  if ((s = attn_launch(a, w.attn_ws, w.attn_ws_bytes, st, err))) return s;
  // 4. h = x + W_o attn  (straight into y when there is no FFN)
  p = ProjArgs{};
  p.W = &L->w_o;
  p.x = w.attn;
  p.x_dtype = act;
  p.n_rows = n;
  p.y = F > 0 ? (void*)w.h : (void*)y;
  p.out_dtype = PKD_F32;
  p.residual = x;
  const bool need_h_bf16 =
      F > 0 && bf && !(tiled_family(L->w_gate_up.family) && L->w_gate_up.dtype == PKD_FP8_E4M3);
  p.y_bf16 = need_h_bf16 ? w.h_in : nullptr;
  if ((s = proj_launch(p, w.proj_ws, w.proj_ws_bytes, st, err))) return s;
  if (F == 0) return ok(err);
  // 5. a = silu(W_gate h) * (W_up h)  (norm: gain in W_gate_up, both halves
  //    times 1/rms(h) before the silu)
  if (norm && (s = rms_factor_launch(w.h, n, D, L->norm_eps, w.inv_h, nullptr, st, err))) return s;
  auto in2 = proj_in(L->w_gate_up, w.h, w.h_in);
  p = ProjArgs{};
  p.W = &L->w_gate_up;
  p.x = in2.first;
  p.x_dtype = in2.second;
  p.n_rows = n;
  p.y = w.a;
  p.out_dtype = act;
  p.silu_pair = 1;
  p.row_scale = norm ? w.inv_h : nullptr;
  if ((s = proj_launch(p, w.proj_ws, w.proj_ws_bytes, st, err))) return s;
  // 6. y = h + W_down a
  p = ProjArgs{};
  p.W = &L->w_down;
  p.x = w.a;
  p.x_dtype = act;
  p.n_rows = n;
  p.y = y;
  p.out_dtype = PKD_F32;
  p.residual = w.h;
  return proj_launch(p, w.proj_ws, w.proj_ws_bytes, st, err);
}

}  // extern "C"
