// Host side of the C ABI: descriptor validation, workspace planning and the
// launch sequence.  Validation and planning touch no device, so they can be
// exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "slikl.h"
#include "slikl_internal.h"
#include "scale_block.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int head_tile(int64_t group) { return group <= 32 ? 32 : (group <= 64 ? 64 : 128); }

int64_t rows_q(const slikl_desc *d) { return d->layout_q == SLIKL_LAYOUT_BSND ? d->batch * d->s1 : d->s1; }
int64_t rows_k(const slikl_desc *d) { return d->layout_k == SLIKL_LAYOUT_BSND ? d->batch * d->s2 : d->s2; }
// longest sequence of a side: S1 / S2 for BSND, the given maximum for TND (0 = not given)
int64_t len_q(const slikl_desc *d) { return d->layout_q == SLIKL_LAYOUT_BSND ? d->s1 : d->max_seqlen_q; }
int64_t len_k(const slikl_desc *d) { return d->layout_k == SLIKL_LAYOUT_BSND ? d->s2 : d->max_seqlen_k; }
bool any_tnd(const slikl_desc *d) { return d->layout_q == SLIKL_LAYOUT_TND || d->layout_k == SLIKL_LAYOUT_TND; }
// 32-key tiles per wave of the dense dK kernel: the kernel fetches a query row's q once
// per key block that its named keys meet.  Blocks of twice the keys halve those fetches
// where they dominate: when q is too large to stay in the on-die caches (more than 128
// MiB), or when rows name few keys of the blocks they meet (top-k lists of at most an
// eighth of the longest key sequence: 4 batches of 8192 rows, top-k 512, dK 3.5 ->
// 2.1 ms; one 4096-row sequence with top-k 2048 runs better with 128-key blocks).
int dense_kt(const slikl_desc *d) {
    const bool big_q = (double)rows_q(d) * d->n1 * d->d * 2.0 > 128.0 * (1 << 20);
    const bool sparse_rows = len_k(d) >= 8 * d->topk;
    return big_q || sparse_rows ? 2 : 1;
}

// Field checks of the operator page's constraints section (dtypes, layouts,
// cuSeqLens required for TND) and of this library's limits (N1 <= 128,
// topk <= 2048 as for the 950-class products; D in {32, 64, 128}).
// Whether the dense dK strategy can take this problem: the longest sequence of each
// side known (BSND, or TND with its maximum given), keys addressed with 32-bit byte
// offsets (< 2^31 bytes) and key rows below 2^24 (24-bit multiplies; exact in fp32).
bool dense_fits(const slikl_desc *d) {
    // the 64-head fused kernel (head groups up to 64) addresses key rows as
    // buffer records, whose stride field holds 14 bits
    const bool rows_ok = head_tile(d->n2 > 0 ? d->n1 / d->n2 : 1) > 64 || (int64_t)d->n2 * d->d * 2 < 16384;
    return len_q(d) > 0 && len_k(d) > 0 && rows_ok &&
           (double)rows_k(d) * d->n2 * d->d * 2.0 < 2147483648.0 && (double)rows_k(d) < 16777216.0;
}

// The key-sorted dK runs through the 64-head kernel's slot records (head groups up to
// 64, key rows within its 14-bit record stride); its bin prefix is one two-level scan.
bool sorted_fits(const slikl_desc *d) {
    // the 64-head kernel (head groups up to 64) addresses key rows as buffer records,
    // whose stride field holds 14 bits
    if (head_tile(d->n2 > 0 ? d->n1 / d->n2 : 1) <= 64 && (int64_t)d->n2 * d->d * 2 >= 16384) return false;
    // record indices are 32-bit; the sort loops step past the last record by up to 4096
    if ((double)rows_q(d) * d->n2 * d->topk >= 2147483648.0 - 65536.0) return false;
    const slikl::SortGeometry g = slikl::sorted_geometry(rows_q(d) * d->n2 * d->topk, rows_k(d) * d->n2);
    return g.nbuckets <= slikl::kSortBucketsMax && g.scan_nb <= 8192;
}

slikl_status validate(const slikl_desc *d) {
    if (!d) return SLIKL_ERR_NULLPTR;
    if (d->layout_q != SLIKL_LAYOUT_BSND && d->layout_q != SLIKL_LAYOUT_TND) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_k != SLIKL_LAYOUT_BSND && d->layout_k != SLIKL_LAYOUT_TND) return SLIKL_ERR_PARAM_INVALID;
    if (d->dtype != SLIKL_DTYPE_F16 && d->dtype != SLIKL_DTYPE_BF16) return SLIKL_ERR_PARAM_INVALID;
    if (d->deterministic != 0 && d->deterministic != 1) return SLIKL_ERR_PARAM_INVALID;
    if (d->split_mode != SLIKL_SPLIT_WEIGHTED && d->split_mode != SLIKL_SPLIT_ROWS) return SLIKL_ERR_PARAM_INVALID;
    if (d->dk_mode < SLIKL_DK_AUTO || d->dk_mode > SLIKL_DK_SORTED) return SLIKL_ERR_PARAM_INVALID;
    if (d->num_parts < 0 || d->num_parts > SLIKL_MAX_PARTS) return SLIKL_ERR_PARAM_INVALID;
    if (d->batch <= 0 || d->batch > INT32_MAX - 1) return SLIKL_ERR_PARAM_INVALID;
    if (d->n1 < 1 || d->n1 > 128) return SLIKL_ERR_PARAM_INVALID;
    if (d->n2 < 1 || d->n1 % d->n2 != 0) return SLIKL_ERR_PARAM_INVALID;
    if (d->d != 32 && d->d != 64 && d->d != 128) return SLIKL_ERR_PARAM_INVALID;
    if (d->topk < 1 || d->topk > 2048) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_q == SLIKL_LAYOUT_TND && !d->cu_seqlens_q) return SLIKL_ERR_NULLPTR;
    if (d->layout_k == SLIKL_LAYOUT_TND && !d->cu_seqlens_k) return SLIKL_ERR_NULLPTR;
    if (d->layout_q == SLIKL_LAYOUT_BSND ? d->s1 <= 0 : d->s1 < 0) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_k == SLIKL_LAYOUT_BSND ? d->s2 <= 0 : d->s2 < 0) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_q == SLIKL_LAYOUT_TND && (d->max_seqlen_q < 0 || d->max_seqlen_q > INT32_MAX))
        return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_k == SLIKL_LAYOUT_TND && (d->max_seqlen_k < 0 || d->max_seqlen_k > INT32_MAX))
        return SLIKL_ERR_PARAM_INVALID;
    // sizes that the kernels index with 32-bit values
    const int64_t lim = (int64_t)INT32_MAX;
    if (d->layout_q == SLIKL_LAYOUT_BSND && d->s1 > lim / d->batch) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_k == SLIKL_LAYOUT_BSND && d->s2 > lim / d->batch) return SLIKL_ERR_PARAM_INVALID;
    // every tensor must have fewer than 2^31 elements (32-bit offsets in the kernels)
    const int64_t t1 = rows_q(d), t2 = rows_k(d);
    if (t1 > lim / (d->n1 * d->d) || t1 > lim / (d->n2 * d->topk)) return SLIKL_ERR_PARAM_INVALID;
    if (t2 > lim / (d->n2 * d->d)) return SLIKL_ERR_PARAM_INVALID;
    if (d->dk_mode == SLIKL_DK_DENSE && !dense_fits(d)) return SLIKL_ERR_UNSUPPORTED;
    if (d->dk_mode == SLIKL_DK_SORTED && !sorted_fits(d)) return SLIKL_ERR_UNSUPPORTED;
    return SLIKL_OK;
}

// Resolved dK strategy: 0 fp32 atomics, 1 int64 fixed-point atomics
// (deterministic), 2 dense records + key-major kernel (deterministic).
int dk_strategy(const slikl_desc *d) {
    const bool fits = dense_fits(d);
    if (d->dk_mode == SLIKL_DK_DENSE && fits) return 2;
    if (d->dk_mode == SLIKL_DK_SORTED) return d->deterministic ? 1 : 0;
    // AUTO: the dense kernels cost about one (row, 128-key block) step per 128 keys of
    // a row's named range (at most S2), the scatter about one atomic row per valid
    // slot, dearer in fixed point (deterministic) and under contention on shared keys:
    // dense when S2 <= 16 topk, or S2 <= 32 topk when deterministic.  Below 2048 units
    // the dense strategy's extra launches outweigh the atomics it saves.
    const int64_t ratio = d->deterministic ? 32 : 16;
    if (d->dk_mode == SLIKL_DK_AUTO && fits && len_k(d) <= ratio * d->topk && rows_q(d) * d->n2 >= 2048) {
        // the dense records are sized [units, longest key sequence]; keep them modest
        const double bytes = (double)rows_q(d) * d->n2 * len_k(d) * 4.0 * (1 + head_tile(d->n1 / d->n2) / 32);
        if (bytes <= 8.0 * (1ull << 30)) return 2;
    }
    return d->deterministic ? 1 : 0;
}

// The key-sorted variant of the scatter strategy: every valid slot's part written once
// as a row of a buffer (16-bit integers with a per-slot multiplier, or fp32 when a key
// takes many parts), then summed per key through a key-sorted record list.
// Asked for explicitly (SORTED), or taken by AUTO where the dense strategy is not and
// there are at least 2048 units (below that its extra launches cost more than the
// atomics they save) and the parts buffer fits in 8 GiB.  Measured on 8192 query rows
// over 131072 keys (S2 = 64 topk, 32 heads): 5.0 ms against 6.9 ms with fp32 atomics,
// 5.4 against 12.1 ms when deterministic.
bool sorted_dk(const slikl_desc *d) {
    if (d->dk_mode == SLIKL_DK_SORTED) return true;      // validate checked sorted_fits
    if (d->dk_mode != SLIKL_DK_AUTO || dk_strategy(d) == 2 || !sorted_fits(d)) return false;
    const double units = (double)rows_q(d) * d->n2;
    return units >= 2048 && units * d->topk * d->d * 4.0 <= 8.0 * (1ull << 30);
}

// Per-unit overhead of the WEIGHTED split for the resolved dK strategy (the sorted
// strategy runs the dense strategy's fused kernel).
int unit_overhead(const slikl_desc *d) {
    return dk_strategy(d) == 2 || sorted_dk(d) ? SLIKL_UNIT_OVERHEAD_DENSE : SLIKL_UNIT_OVERHEAD;
}

// Dense dK task geometry: key blocks per (batch, key head), row chunk length and
// count (at most 256 chunks per batch), and the most tasks the table can hold.
void dense_dk_geometry(const slikl_desc *d, int *nkb, int *chunk, int *nch, int *max_tasks) {
    const int64_t kb = slikl::dense_dk_keys_per_block(dense_kt(d));
    *nkb = (int)((len_k(d) + kb - 1) / kb);
    const int64_t c = (len_q(d) + 255) / 256;
    *chunk = (int)(c < 16 ? 16 : c);
    *nch = (int)((len_q(d) + *chunk - 1) / *chunk);
    *max_tasks = slikl::kDkSlotsMax + (int)(d->batch * d->n2) * *nkb;
}

slikl::WorkspacePlan plan(const slikl_desc *d) {
    slikl::WorkspacePlan p{};
    const int64_t t1 = rows_q(d), t2 = rows_k(d);
    const size_t U = (size_t)t1 * (size_t)d->n2;
    const int mode = dk_strategy(d);
    p.mode = mode;
    const size_t acc_elem = mode == 1 ? 8 : 4;
    size_t off = 0;
    p.acc_off = off;
    p.acc_bytes = mode == 2 ? 0 : (size_t)t2 * (size_t)d->n2 * (size_t)d->d * acc_elem;
    off = align_up(off + p.acc_bytes);
    p.meta_off = off;
    off = align_up(off + SLIKL_METADATA_INTS * sizeof(int32_t));
    p.prefix_off = off;
    p.prefix_bytes = (U + 1) * sizeof(int64_t);
    off = align_up(off + p.prefix_bytes);
    p.flags_off = off;
    off = align_up(off + (size_t)slikl::kMetaCountBlocksMax * 4);
    p.scale_off = off;
    off = align_up(off + slikl::kScaleBlockBytes);
    p.zero_off = off;
    off = align_up(off + 256);
    p.k16_off = off;
    p.k16_bytes = d->dtype == SLIKL_DTYPE_BF16 ? (size_t)t2 * (size_t)d->n2 * (size_t)d->d * 2 : 0;
    off = align_up(off + p.k16_bytes);
    if (mode == 2) {
        const size_t s2 = (size_t)len_k(d), nh = (size_t)head_tile(d->n1 / d->n2) / 32;
        dense_dk_geometry(d, &p.dk_nkb, &p.dk_chunk, &p.dk_nch, &p.dk_max_tasks);
        const size_t nbg = (size_t)d->batch * (size_t)d->n2;
        p.dimap_off = off;
        p.dimap_bytes = U * s2 * 4;
        off = align_up(off + p.dimap_bytes);
        p.maskmap_off = off;
        off = align_up(off + U * s2 * nh * 4);
        p.range_off = off;
        off = align_up(off + U * 8);
        p.q16_off = off;
        off = align_up(off + (d->dtype == SLIKL_DTYPE_BF16 ? (size_t)t1 * (size_t)d->n1 * (size_t)d->d * 2 : 0));
        p.wrec_off = off;
        off = align_up(off + U * (size_t)slikl::wrec_bytes(head_tile(d->n1 / d->n2)));
        p.part_off = off;
        off = align_up(off + (size_t)p.dk_max_tasks * slikl::dense_dk_keys_per_block(dense_kt(d)) * (size_t)d->d * 4);
        p.kbdiff_off = off;
        p.kbdiff_bytes = nbg * (size_t)p.dk_nch * (size_t)(p.dk_nkb + 1) * 4;
        off = align_up(off + p.kbdiff_bytes);
        p.tasks_off = off;
        off = align_up(off + (size_t)p.dk_max_tasks * 16);
        p.kbtasks_off = off;
        off = align_up(off + nbg * (size_t)p.dk_nkb * 16);
        p.ntasks_off = off;
        off = align_up(off + 16);
        p.rowinfo_off = off;
        off = align_up(off + (any_tnd(d) ? (size_t)t1 * 16 : 0));
    }
    if (mode != 2 && sorted_dk(d)) {
        const size_t nslot = U * (size_t)d->topk;
        const size_t nh = (size_t)head_tile(d->n1 / d->n2) / 32;
        p.srec_key_off = off;
        off = align_up(off + nslot * 4);
        p.srec_dI_off = off;
        off = align_up(off + nslot * 4);
        p.srec_mask_off = off;
        off = align_up(off + nslot * nh * 4);
        p.srec_cnt_off = off;
        off = align_up(off + U * 4);
        const size_t nbins = (size_t)t2 * (size_t)d->n2;
        const slikl::SortGeometry g = slikl::sorted_geometry((int64_t)nslot, (int64_t)nbins);
        p.sorted = true;
        p.hist_off = off;
        off = align_up(off + ((size_t)g.hist_n + 1) * 4);
        p.sblk_off = off;
        off = align_up(off + (size_t)g.scan_nb * 4);
        p.tmp_off = off;
        off = align_up(off + nslot * 8);
        p.list_off = off;
        off = align_up(off + nslot * 4);
        p.bin_off = off;
        off = align_up(off + (nbins + 1) * 4);
        p.parts_off = off;
        off = align_up(off + nslot * (size_t)d->d * 4);
        p.rowinfo_off = off;
        off = align_up(off + (any_tnd(d) ? (size_t)t1 * 16 : 0));
    }
    p.total = off;
    return p;
}

slikl::Problem problem(const slikl_desc *d) {
    slikl::Problem pb{};
    pb.t1 = rows_q(d);
    pb.t2 = rows_k(d);
    pb.s1 = d->s1;
    pb.s2 = d->s2;
    pb.batch = (int32_t)d->batch;
    pb.n1 = (int32_t)d->n1;
    pb.n2 = (int32_t)d->n2;
    pb.group = (int32_t)(d->n1 / d->n2);
    pb.d = (int32_t)d->d;
    pb.topk = (int32_t)d->topk;
    pb.layout_q = d->layout_q;
    pb.layout_k = d->layout_k;
    pb.cu_q = d->layout_q == SLIKL_LAYOUT_TND ? d->cu_seqlens_q : nullptr;
    pb.cu_k = d->layout_k == SLIKL_LAYOUT_TND ? d->cu_seqlens_k : nullptr;
    pb.max_q = d->layout_q == SLIKL_LAYOUT_TND ? d->max_seqlen_q : 0;
    pb.max_k = d->layout_k == SLIKL_LAYOUT_TND ? d->max_seqlen_k : 0;
    pb.kl = d->kl_loss;
    pb.used_q = d->layout_q == SLIKL_LAYOUT_TND ? d->seq_used_q : nullptr;
    pb.used_k = d->layout_k == SLIKL_LAYOUT_TND ? d->seq_used_k : nullptr;
    return pb;
}

slikl_status resolve_parts(const slikl_desc *d, int32_t *parts) {
    if (d->num_parts > 0) {
        *parts = d->num_parts;
        return SLIKL_OK;
    }
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SLIKL_ERR_LAUNCH;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return SLIKL_ERR_LAUNCH;
    const int mode = dk_strategy(d);
    const int hp = head_tile(d->n1 / d->n2);
    const bool f16 = d->dtype == SLIKL_DTYPE_F16;
    int per_cu = mode == 2 || sorted_dk(d)
                     ? slikl::grad_dense_blocks_per_cu(hp, (int)d->d, f16, slikl::dense64_cap(d->topk),
                                                       (int)(d->n1 / d->n2))
                     : slikl::grad_fused_blocks_per_cu(hp, (int)d->d, f16, mode);
    int64_t p = (int64_t)cus * per_cu;
    // with TND queries the 64-head fused kernel takes its parts from a counter, four per
    // workgroup on average: sequences of different lengths leave whole-part splits
    // uneven (8 sequences of 512..8192 rows, 64 heads: fused kernel 4.49 -> 4.06 ms);
    // BSND rows keep one part per workgroup, where the counter's traffic cost more than
    // it balanced (one 4096-row sequence, 64 heads, top-k 2048: 408 -> 465 us)
    if ((mode == 2 || sorted_dk(d)) && hp <= 64 && d->layout_q == SLIKL_LAYOUT_TND) p *= 4;
    if (p > SLIKL_MAX_PARTS) p = SLIKL_MAX_PARTS;
    if (p < 1) p = 1;
    *parts = (int32_t)p;
    return SLIKL_OK;
}

}  // namespace

extern "C" {

const char *slikl_status_string(slikl_status s) {
    switch (s) {
        case SLIKL_OK: return "ok";
        case SLIKL_ERR_NULLPTR: return "a required pointer is NULL";
        case SLIKL_ERR_PARAM_INVALID: return "a descriptor field is out of range";
        case SLIKL_ERR_UNSUPPORTED: return "configuration not supported";
        case SLIKL_ERR_WORKSPACE: return "workspace missing or too small";
        case SLIKL_ERR_LAUNCH: return "HIP launch or device query failed";
    }
    return "unknown status";
}

slikl_status slikl_grad_workspace_size(const slikl_desc *desc, size_t *bytes) {
    if (!desc || !bytes) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    *bytes = plan(desc).total;
    return SLIKL_OK;
}

slikl_status slikl_grad_parts(const slikl_desc *desc, int32_t *parts) {
    if (!desc || !parts) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    return resolve_parts(desc, parts);
}

slikl_status slikl_grad_unit_overhead(const slikl_desc *desc, int32_t *overhead) {
    if (!desc || !overhead) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    *overhead = unit_overhead(desc);
    return SLIKL_OK;
}

slikl_status slikl_grad_dk_strategy(const slikl_desc *desc, int32_t *strategy) {
    if (!desc || !strategy) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    *strategy = dk_strategy(desc) == 2 ? SLIKL_DK_DENSE : sorted_dk(desc) ? SLIKL_DK_SORTED : SLIKL_DK_SCATTER;
    return SLIKL_OK;
}

slikl_status slikl_grad_metadata(const slikl_desc *desc, const int32_t *sparse_indices, int32_t *metadata,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    if (!desc || !metadata) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    if (desc->split_mode == SLIKL_SPLIT_WEIGHTED && !sparse_indices && rows_q(desc) > 0)
        return SLIKL_ERR_NULLPTR;
    slikl::WorkspacePlan wp = plan(desc);
    if (!workspace || workspace_bytes < wp.total) return SLIKL_ERR_WORKSPACE;
    int32_t parts = 0;
    st = resolve_parts(desc, &parts);
    if (st != SLIKL_OK) return st;
    slikl::Problem pb = problem(desc);
    pb.idx = sparse_indices;
    if ((uintptr_t)workspace % 256 != 0) return SLIKL_ERR_WORKSPACE;
    hipError_t e = slikl::launch_metadata(pb, parts, desc->split_mode, unit_overhead(desc), metadata,
                                          (int64_t *)((char *)workspace + wp.prefix_off),
                                          (int32_t *)((char *)workspace + wp.flags_off), (hipStream_t)stream);
    return e == hipSuccess ? SLIKL_OK : SLIKL_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Optional per-phase timing with HIP events recorded on the launch stream.
struct PhaseEvents {
    bool on = false;
    hipEvent_t ev[2 * SLIKL_PHASES] = {};
    bool used[SLIKL_PHASES] = {};
    hipStream_t s = nullptr;
    float extra_fill_ms = 0.f;      // fills timed outside these events (dense index lists)
    bool init(hipStream_t st) {
        s = st;
        on = true;
        for (int i = 0; i < 2 * SLIKL_PHASES; ++i)
            if (hipEventCreate(&ev[i]) != hipSuccess) return false;
        return true;
    }
    void begin(int p) {
        if (on) hipEventRecord(ev[2 * p], s);
    }
    void end(int p) {
        if (on) {
            hipEventRecord(ev[2 * p + 1], s);
            used[p] = true;
        }
    }
    bool collect(float *ms) {
        bool ok = true;
        for (int p = 0; p < SLIKL_PHASES; ++p) {
            ms[p] = 0.f;
            if (!used[p]) continue;
            if (hipEventSynchronize(ev[2 * p + 1]) != hipSuccess ||
                hipEventElapsedTime(&ms[p], ev[2 * p], ev[2 * p + 1]) != hipSuccess)
                ok = false;
        }
        return ok;
    }
    ~PhaseEvents() {
        for (int i = 0; i < 2 * SLIKL_PHASES; ++i)
            if (ev[i]) hipEventDestroy(ev[i]);
    }
};

slikl_status grad_impl(const slikl_desc *desc, const void *q, const void *k, const float *w,
                       const int32_t *sparse_indices, const float *attn_softmax_l1norm,
                       const int32_t *metadata, void *dq, void *dk, float *dw, float *softmax_out,
                       void *workspace, size_t workspace_bytes, void *stream, PhaseEvents &pe) {
    if (!desc) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    const int64_t t1 = rows_q(desc), t2 = rows_k(desc);
    if (t1 > 0 && (!q || !w || !sparse_indices || !attn_softmax_l1norm || !dq || !dw || !softmax_out))
        return SLIKL_ERR_NULLPTR;
    if (t2 > 0 && (!k || !dk)) return SLIKL_ERR_NULLPTR;
    slikl::WorkspacePlan wp = plan(desc);
    if (!workspace || workspace_bytes < wp.total || (uintptr_t)workspace % 256 != 0)
        return SLIKL_ERR_WORKSPACE;
    // 16-byte vector loads / stores of the 16-bit tensors
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)dq | (uintptr_t)dk) % 16 != 0)
        return SLIKL_ERR_PARAM_INVALID;
    int32_t parts = 0;
    st = resolve_parts(desc, &parts);
    if (st != SLIKL_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    if (pe.on && !pe.init(s)) return SLIKL_ERR_LAUNCH;
    char *ws = (char *)workspace;
    const bool f16 = desc->dtype == SLIKL_DTYPE_F16;

    slikl::Problem pb = problem(desc);
    pb.q = (const uint16_t *)q;
    pb.k = (const uint16_t *)k;
    pb.w = w;
    pb.idx = sparse_indices;
    pb.p = attn_softmax_l1norm;
    pb.dq = (uint16_t *)dq;
    pb.dk = (uint16_t *)dk;
    pb.dw = dw;
    pb.y = softmax_out;
    pb.dk_acc = ws + wp.acc_off;
    pb.det_scale = (const float *)(ws + wp.scale_off);
    pb.k16 = f16 ? pb.k : (const uint16_t *)(ws + wp.k16_off);
    pb.zero16 = (const uint16_t *)(ws + wp.zero_off);
    const int mode = wp.mode;
    const bool s8 = wp.sorted;          // 64-head kernel writing slot records
    if (s8) {
        pb.srec_key = (int32_t *)(ws + wp.srec_key_off);
        pb.srec_dI = (float *)(ws + wp.srec_dI_off);
        pb.srec_mask = (uint32_t *)(ws + wp.srec_mask_off);
        pb.srec_cnt = (int32_t *)(ws + wp.srec_cnt_off);
        const slikl::SortGeometry g = slikl::sorted_geometry(t1 * desc->n2 * desc->topk, t2 * desc->n2);
        pb.sort_hist = (int32_t *)(ws + wp.hist_off);
        pb.sort_blk = (int32_t *)(ws + wp.sblk_off);
        pb.sort_tmp = (int32_t *)(ws + wp.tmp_off);
        pb.sort_list = (int32_t *)(ws + wp.list_off);
        pb.bin_start = (int32_t *)(ws + wp.bin_off);
        pb.dk_parts = ws + wp.parts_off;
        pb.sort_maxref = (int32_t *)(ws + wp.scale_off) + 8;      // in the zeroed scale block
        pb.sort_shift = g.shift;
        pb.sort_nbuckets = g.nbuckets;
        pb.sort_tile = g.tile;
        pb.sort_nblk = g.nblk;
        pb.s2max = t2;                  // no record width: key lengths are not clamped
        pb.rowinfo = any_tnd(desc) ? (const slikl::i32x4 *)(ws + wp.rowinfo_off) : nullptr;
    }
    if (mode == 2) {
        pb.dI_map = (int32_t *)(ws + wp.dimap_off);
        pb.mask_map = (uint32_t *)(ws + wp.maskmap_off);
        pb.row_range = (int32_t *)(ws + wp.range_off);
        pb.q16 = (uint16_t *)(ws + wp.q16_off);
        pb.wrec = (uint8_t *)(ws + wp.wrec_off);
        pb.dk_part = (float *)(ws + wp.part_off);
        pb.kb_diff = (int32_t *)(ws + wp.kbdiff_off);
        pb.dk_tasks = (int32_t *)(ws + wp.tasks_off);
        pb.kb_tasks = (int32_t *)(ws + wp.kbtasks_off);
        pb.dk_ntasks = (int32_t *)(ws + wp.ntasks_off);
        pb.dk_kb = slikl::dense_dk_keys_per_block(dense_kt(desc));
        pb.dk_nkb = wp.dk_nkb;
        pb.dk_chunk = wp.dk_chunk;
        pb.dk_nch = wp.dk_nch;
        pb.dk_max_tasks = wp.dk_max_tasks;
        {
            int dev = 0, cus = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
                return SLIKL_ERR_LAUNCH;
            int64_t slots = (int64_t)cus * slikl::dense_dk_wgs_per_cu(head_tile(pb.group), (int)desc->d, dense_kt(desc));
            pb.dk_slots = (int)(slots > slikl::kDkSlotsMax ? slikl::kDkSlotsMax : slots);
        }
        pb.s2max = len_k(desc);
        pb.rowinfo = any_tnd(desc) ? (const slikl::i32x4 *)(ws + wp.rowinfo_off) : nullptr;
    }

    hipError_t e = hipSuccess;
    if (!metadata) {
        int32_t *md = (int32_t *)(ws + wp.meta_off);
        pe.begin(SLIKL_PHASE_METADATA);
        e = slikl::launch_metadata(pb, parts, desc->split_mode, unit_overhead(desc), md,
                                   (int64_t *)(ws + wp.prefix_off), (int32_t *)(ws + wp.flags_off), s);
        pe.end(SLIKL_PHASE_METADATA);
        if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
        metadata = md;
    }
    pb.metadata = metadata;
    pb.part_ctr = (int32_t *)(ws + wp.scale_off) + 12;        // in the zeroed scale block
    pe.begin(SLIKL_PHASE_FILL);
    {
        // the dense dI rows are zeroed by the fused kernel, each over the key blocks
        // its unit's named keys meet
        slikl::ZeroRanges zr{};
        zr.add(pb.dk_acc, wp.acc_bytes);
        zr.add(ws + wp.scale_off, slikl::kScaleBlockBytes);
        zr.add(ws + wp.zero_off, 256);
        if (mode == 2) zr.add(pb.kb_diff, wp.kbdiff_bytes);
        e = slikl::launch_zero_ranges(zr, s);
        if (e == hipSuccess && pb.rowinfo)
            e = slikl::launch_rowinfo(pb, (slikl::i32x4 *)pb.rowinfo, s);
    }
    pe.end(SLIKL_PHASE_FILL);
    if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
    if (!f16 && t2 > 0) {
        pe.begin(SLIKL_PHASE_KEY_COPY);
        e = slikl::launch_k_to_f16(pb, (uint16_t *)(ws + wp.k16_off), (float *)(ws + wp.scale_off), s);
        pe.end(SLIKL_PHASE_KEY_COPY);
        if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
    }
    if (mode == 1) {
        pe.begin(SLIKL_PHASE_DET_SCALE);
        e = slikl::launch_det_scale(pb, f16, (float *)(ws + wp.scale_off), s);
        pe.end(SLIKL_PHASE_DET_SCALE);
        if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
    }
    if (t1 > 0) {
        pe.begin(SLIKL_PHASE_FUSED);
        e = mode == 2 || s8 ? slikl::launch_grad_dense(pb, head_tile(pb.group), f16, slikl::dense64_cap(desc->topk),
                                                       parts, s8, s)
                            : slikl::launch_grad_fused(pb, head_tile(pb.group), f16, mode, parts, s);
        pe.end(SLIKL_PHASE_FUSED);
        if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
        if (s8) {
            pe.begin(SLIKL_PHASE_DK_PREP);
            e = slikl::launch_sorted_prepare(pb, s);
            pe.end(SLIKL_PHASE_DK_PREP);
            if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
            pe.begin(SLIKL_PHASE_DK);
            e = slikl::launch_scatter_dk(pb, head_tile(pb.group), f16, s);
            pe.end(SLIKL_PHASE_DK);
            if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
            pe.begin(SLIKL_PHASE_DK_REDUCE);
            e = slikl::launch_sorted_reduce(pb, mode == 1, s);
            pe.end(SLIKL_PHASE_DK_REDUCE);
            if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
        }
    }
    if (mode == 2) {
        pe.begin(SLIKL_PHASE_DK_PREP);
        e = slikl::launch_dense_dk_tasks(pb, s);
        pe.end(SLIKL_PHASE_DK_PREP);
        if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
        pe.begin(SLIKL_PHASE_DK);
        e = slikl::launch_dense_dk(pb, head_tile(pb.group), f16, s);
        pe.end(SLIKL_PHASE_DK);
        if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
        pe.begin(SLIKL_PHASE_DK_FINAL);
        e = slikl::launch_dense_dk_reduce(pb, f16, s);
        pe.end(SLIKL_PHASE_DK_FINAL);
        if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
        return SLIKL_OK;
    }
    pe.begin(SLIKL_PHASE_DK_FINAL);
    e = slikl::launch_finalize_dk(pb, f16, mode == 1, s);
    pe.end(SLIKL_PHASE_DK_FINAL);
    if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
    return SLIKL_OK;
}

}  // namespace

extern "C" {

slikl_status slikl_grad(const slikl_desc *desc, const void *q, const void *k, const float *w,
                        const int32_t *sparse_indices, const float *attn_softmax_l1norm,
                        const int32_t *metadata, void *dq, void *dk, float *dw, float *softmax_out,
                        void *workspace, size_t workspace_bytes, void *stream) {
    PhaseEvents pe;
    return grad_impl(desc, q, k, w, sparse_indices, attn_softmax_l1norm, metadata, dq, dk, dw, softmax_out,
                     workspace, workspace_bytes, stream, pe);
}

slikl_status slikl_grad_profiled(const slikl_desc *desc, const void *q, const void *k, const float *w,
                                 const int32_t *sparse_indices, const float *attn_softmax_l1norm,
                                 const int32_t *metadata, void *dq, void *dk, float *dw, float *softmax_out,
                                 void *workspace, size_t workspace_bytes, void *stream, float *phase_ms) {
    if (!phase_ms) return SLIKL_ERR_NULLPTR;
    PhaseEvents pe;
    pe.on = true;
    slikl_status st = grad_impl(desc, q, k, w, sparse_indices, attn_softmax_l1norm, metadata, dq, dk, dw,
                                softmax_out, workspace, workspace_bytes, stream, pe);
    if (st != SLIKL_OK) return st;
    return pe.collect(phase_ms) ? SLIKL_OK : SLIKL_ERR_LAUNCH;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The dense sibling operator: slikl_grad over index lists of the visible keys.
// ---------------------------------------------------------------------------
namespace {

// The sparse descriptor the dense call runs (topk = the dense axis L), validated.
slikl_status dense_sparse_desc(const slikl_dense_desc *d, slikl_desc *sd) {
    if (!d) return SLIKL_ERR_NULLPTR;
    if (d->mask_mode != 0 && d->mask_mode != 3) return SLIKL_ERR_PARAM_INVALID;
    if (d->cmp_ratio < 1 || d->cmp_ratio > 128) return SLIKL_ERR_PARAM_INVALID;
    if (d->cmp_ratio != 1) return SLIKL_ERR_UNSUPPORTED;
    if (d->base.seq_used_q || d->base.seq_used_k) return SLIKL_ERR_UNSUPPORTED;
    *sd = d->base;
    const int64_t L = sd->layout_k == SLIKL_LAYOUT_BSND ? sd->s2 : sd->max_seqlen_k;
    if (L < 1) return SLIKL_ERR_PARAM_INVALID;
    if (L > 2048) return SLIKL_ERR_UNSUPPORTED;
    sd->topk = L;
    return validate(sd);
}

size_t dense_idx_off(const slikl_desc *sd) { return align_up(plan(sd).total); }
size_t dense_ws_bytes(const slikl_desc *sd) {
    return dense_idx_off(sd) + align_up((size_t)rows_q(sd) * (size_t)sd->n2 * (size_t)sd->topk * 4);
}

}  // namespace

extern "C" {

slikl_status slikl_dense_grad_workspace_size(const slikl_dense_desc *desc, size_t *bytes) {
    if (!desc || !bytes) return SLIKL_ERR_NULLPTR;
    slikl_desc sd;
    slikl_status st = dense_sparse_desc(desc, &sd);
    if (st != SLIKL_OK) return st;
    *bytes = dense_ws_bytes(&sd);
    return SLIKL_OK;
}

slikl_status slikl_dense_grad_metadata(const slikl_dense_desc *desc, int32_t *metadata, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    if (!desc || !metadata) return SLIKL_ERR_NULLPTR;
    slikl_desc sd;
    slikl_status st = dense_sparse_desc(desc, &sd);
    if (st != SLIKL_OK) return st;
    if (!workspace || workspace_bytes < dense_ws_bytes(&sd) || (uintptr_t)workspace % 256 != 0)
        return SLIKL_ERR_WORKSPACE;
    int32_t *idx = (int32_t *)((char *)workspace + dense_idx_off(&sd));
    slikl::Problem pb = problem(&sd);
    hipError_t e = slikl::launch_dense_index(pb, idx, desc->mask_mode, (int)sd.topk, (hipStream_t)stream);
    if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
    return slikl_grad_metadata(&sd, idx, metadata, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

slikl_status dense_grad_impl(const slikl_dense_desc *desc, const void *q, const void *k, const float *w,
                             const float *p, const int32_t *metadata, void *dq, void *dk, float *dw, float *y,
                             void *workspace, size_t workspace_bytes, void *stream, PhaseEvents &pe) {
    slikl_desc sd;
    slikl_status st = dense_sparse_desc(desc, &sd);
    if (st != SLIKL_OK) return st;
    if (!workspace || workspace_bytes < dense_ws_bytes(&sd) || (uintptr_t)workspace % 256 != 0)
        return SLIKL_ERR_WORKSPACE;
    int32_t *idx = (int32_t *)((char *)workspace + dense_idx_off(&sd));
    slikl::Problem pb = problem(&sd);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (pe.on) {
        if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return SLIKL_ERR_LAUNCH;
        hipEventRecord(e0, (hipStream_t)stream);
    }
    hipError_t e = slikl::launch_dense_index(pb, idx, desc->mask_mode, (int)sd.topk, (hipStream_t)stream);
    if (pe.on) hipEventRecord(e1, (hipStream_t)stream);
    if (e != hipSuccess) return SLIKL_ERR_LAUNCH;
    st = grad_impl(&sd, q, k, w, rows_q(&sd) > 0 ? idx : nullptr, p, metadata, dq, dk, dw, y, workspace,
                   workspace_bytes, stream, pe);
    if (pe.on) {
        // the index fill is part of the call's fills
        float ms = 0.f;
        if (hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess)
            pe.extra_fill_ms = ms;
        hipEventDestroy(e0);
        hipEventDestroy(e1);
    }
    return st;
}

}  // namespace

extern "C" {

slikl_status slikl_dense_grad(const slikl_dense_desc *desc, const void *q, const void *k, const float *w,
                              const float *attn_softmax_l1norm, const int32_t *metadata, void *dq, void *dk,
                              float *dw, float *softmax_out, void *workspace, size_t workspace_bytes,
                              void *stream) {
    PhaseEvents pe;
    return dense_grad_impl(desc, q, k, w, attn_softmax_l1norm, metadata, dq, dk, dw, softmax_out, workspace,
                           workspace_bytes, stream, pe);
}

slikl_status slikl_dense_grad_profiled(const slikl_dense_desc *desc, const void *q, const void *k,
                                       const float *w, const float *attn_softmax_l1norm,
                                       const int32_t *metadata, void *dq, void *dk, float *dw,
                                       float *softmax_out, void *workspace, size_t workspace_bytes,
                                       void *stream, float *phase_ms) {
    if (!phase_ms) return SLIKL_ERR_NULLPTR;
    PhaseEvents pe;
    pe.on = true;
    slikl_status st = dense_grad_impl(desc, q, k, w, attn_softmax_l1norm, metadata, dq, dk, dw, softmax_out,
                                      workspace, workspace_bytes, stream, pe);
    if (st != SLIKL_OK) return st;
    if (!pe.collect(phase_ms)) return SLIKL_ERR_LAUNCH;
    phase_ms[SLIKL_PHASE_FILL] += pe.extra_fill_ms;
    return SLIKL_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The target distribution p from the main attention.
// ---------------------------------------------------------------------------
namespace {

slikl_status validate_attn_p(const slikl_attn_p_desc *d) {
    if (!d) return SLIKL_ERR_NULLPTR;
    if (d->layout_q != SLIKL_LAYOUT_BSND && d->layout_q != SLIKL_LAYOUT_TND) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_k != SLIKL_LAYOUT_BSND && d->layout_k != SLIKL_LAYOUT_TND) return SLIKL_ERR_PARAM_INVALID;
    if (d->dtype != SLIKL_DTYPE_F16 && d->dtype != SLIKL_DTYPE_BF16) return SLIKL_ERR_PARAM_INVALID;
    if (d->reserved != 0) return SLIKL_ERR_PARAM_INVALID;
    if (d->batch <= 0 || d->batch > INT32_MAX - 1) return SLIKL_ERR_PARAM_INVALID;
    if (d->n2 < 1 || d->heads < 1 || d->heads % d->n2 != 0 || d->heads / d->n2 > 128) return SLIKL_ERR_PARAM_INVALID;
    if (d->d != 64 && d->d != 128 && d->d != 256 && d->d != 512 && d->d != 576) return SLIKL_ERR_PARAM_INVALID;
    if (d->n2 * d->d * 2 >= 16384) return SLIKL_ERR_PARAM_INVALID;     // key record stride: 14 bits
    if (d->topk < 1 || d->topk > 2048) return SLIKL_ERR_PARAM_INVALID;
    if (!(d->scale == d->scale) || d->scale > 3.0e38f || d->scale < -3.0e38f) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_q == SLIKL_LAYOUT_TND && !d->cu_seqlens_q) return SLIKL_ERR_NULLPTR;
    if (d->layout_k == SLIKL_LAYOUT_TND && !d->cu_seqlens_k) return SLIKL_ERR_NULLPTR;
    if (d->layout_q == SLIKL_LAYOUT_BSND ? d->s1 <= 0 : d->s1 < 0) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_k == SLIKL_LAYOUT_BSND ? d->s2 <= 0 : d->s2 < 0) return SLIKL_ERR_PARAM_INVALID;
    const int64_t lim = (int64_t)INT32_MAX;
    if (d->layout_q == SLIKL_LAYOUT_BSND && d->s1 > lim / d->batch) return SLIKL_ERR_PARAM_INVALID;
    if (d->layout_k == SLIKL_LAYOUT_BSND && d->s2 > lim / d->batch) return SLIKL_ERR_PARAM_INVALID;
    const int64_t t1 = d->layout_q == SLIKL_LAYOUT_BSND ? d->batch * d->s1 : d->s1;
    const int64_t t2 = d->layout_k == SLIKL_LAYOUT_BSND ? d->batch * d->s2 : d->s2;
    // 32-bit element offsets in the kernel for the index lists, p and lse; 64-bit for q
    if (t1 > lim / (d->n2 * d->topk) || t1 > lim / d->heads) return SLIKL_ERR_PARAM_INVALID;
    if (t2 > lim / (d->n2 * d->d)) return SLIKL_ERR_PARAM_INVALID;
    return SLIKL_OK;
}

}  // namespace

extern "C" slikl_status slikl_attn_softmax_l1norm(const slikl_attn_p_desc *desc, const void *q_main,
                                                  const void *k_main, const int32_t *sparse_indices,
                                                  const float *lse, float *p, void *stream) {
    slikl_status st = validate_attn_p(desc);
    if (st != SLIKL_OK) return st;
    const int64_t t1 = desc->layout_q == SLIKL_LAYOUT_BSND ? desc->batch * desc->s1 : desc->s1;
    const int64_t t2 = desc->layout_k == SLIKL_LAYOUT_BSND ? desc->batch * desc->s2 : desc->s2;
    if (t1 > 0 && (!q_main || !sparse_indices || !p)) return SLIKL_ERR_NULLPTR;
    if (t2 > 0 && !k_main) return SLIKL_ERR_NULLPTR;
    if (((uintptr_t)q_main | (uintptr_t)k_main) % 16 != 0) return SLIKL_ERR_PARAM_INVALID;
    if (t1 == 0) return SLIKL_OK;
    slikl::AttnPProblem pb{};
    pb.q = (const uint16_t *)q_main;
    pb.k = (const uint16_t *)k_main;
    pb.idx = sparse_indices;
    pb.lse = lse;
    pb.p = p;
    pb.cu_q = desc->layout_q == SLIKL_LAYOUT_TND ? desc->cu_seqlens_q : nullptr;
    pb.cu_k = desc->layout_k == SLIKL_LAYOUT_TND ? desc->cu_seqlens_k : nullptr;
    pb.s1 = desc->s1;
    pb.s2 = desc->s2;
    pb.t1 = t1;
    pb.t2 = t2;
    pb.batch = (int32_t)desc->batch;
    pb.nm = (int32_t)desc->heads;
    pb.n2 = (int32_t)desc->n2;
    pb.hm = (int32_t)(desc->heads / desc->n2);
    pb.dm = (int32_t)desc->d;
    pb.topk = (int32_t)desc->topk;
    pb.layout_q = desc->layout_q;
    pb.layout_k = desc->layout_k;
    pb.scale_log2 = desc->scale * 1.4426950408889634f;
    hipError_t e = slikl::launch_attn_p(pb, desc->dtype == SLIKL_DTYPE_F16, (hipStream_t)stream);
    return e == hipSuccess ? SLIKL_OK : SLIKL_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: its workspace is a fixed device array of
// this library, one copy per GPU, whose device address is looked up once per device.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[SLIKL_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (nullptr on failure).  Called with
// the caller's device current; the address is kept per device.
void *scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// The strategy the no-alloc call runs: the descriptor's own when its workspace fits
// the fixed array; with AUTO, else the scatter strategy (the least workspace).
bool noalloc_desc(const slikl_desc *in, slikl_desc *out) {
    *out = *in;
    if (plan(out).total <= SLIKL_STATIC_SCRATCH_BYTES) return true;
    if (in->dk_mode != SLIKL_DK_AUTO) return false;
    out->dk_mode = SLIKL_DK_SCATTER;
    return plan(out).total <= SLIKL_STATIC_SCRATCH_BYTES;
}

}  // namespace

extern "C" {

slikl_status slikl_grad_noalloc_strategy(const slikl_desc *desc, int32_t *strategy) {
    if (!desc || !strategy) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    slikl_desc d2;
    if (!noalloc_desc(desc, &d2)) return SLIKL_ERR_WORKSPACE;
    *strategy = dk_strategy(&d2) == 2 ? SLIKL_DK_DENSE : sorted_dk(&d2) ? SLIKL_DK_SORTED : SLIKL_DK_SCATTER;
    return SLIKL_OK;
}

slikl_status slikl_grad_noalloc(const slikl_desc *desc, const void *q, const void *k, const float *w,
                                const int32_t *sparse_indices, const float *attn_softmax_l1norm,
                                const int32_t *metadata, void *dq, void *dk, float *dw, float *softmax_out,
                                void *stream) {
    if (!desc) return SLIKL_ERR_NULLPTR;
    slikl_status st = validate(desc);
    if (st != SLIKL_OK) return st;
    slikl_desc d2;
    if (!noalloc_desc(desc, &d2)) return SLIKL_ERR_WORKSPACE;
    // a caller's metadata may have been cut for another strategy: the fused kernels walk
    // whatever parts it holds, and results do not depend on the split
    void *ws = scratch_address();
    if (!ws) return SLIKL_ERR_LAUNCH;
    PhaseEvents pe;
    return grad_impl(&d2, q, k, w, sparse_indices, attn_softmax_l1norm, metadata, dq, dk, dw, softmax_out, ws,
                     SLIKL_STATIC_SCRATCH_BYTES, stream, pe);
}

}  // extern "C"
