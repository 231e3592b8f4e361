// pipeline.hip -- the block-by-block schedule of libeq (host code only).
//
// EntQuant ("Float8@2bits: Entropy Coding Enables Data-Free Model
// Compression", technical summary, section 2, technical component 3) decodes
// each transformer block's weights into a buffer just before the block runs.
// eq_pipeline_run enqueues that schedule for a whole model on two HIP
// streams: each block's decode (eq_decode_dequant_bf16, into one of two bf16
// buffers) on the decode stream, its batch-1 GEMVs (eq_gemv_bf16) on the GEMV
// stream, HIP events between them. Nothing here allocates device memory or
// synchronises with the host.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <vector>

#include "../../include/eq.h"

struct eq_pipeline {
    uint32_t n_blocks;
    uint32_t overlap;  // EQ_PIPELINE_ALTERNATE or EQ_PIPELINE_OVERLAP
    std::vector<hipEvent_t> decoded, consumed;
    hipEvent_t start;  // gemv_stream's position when a run begins
};

extern "C" {

eq_status eq_pipeline_create(uint32_t n_blocks, eq_pipeline **out) {
    if (!out || n_blocks == 0) return EQ_EINVAL;
    eq_pipeline *p = new (std::nothrow) eq_pipeline;
    if (!p) return EQ_ENOMEM;
    p->n_blocks = n_blocks;
    p->overlap = EQ_PIPELINE_ALTERNATE;
    p->decoded.assign(n_blocks, nullptr);
    p->consumed.assign(n_blocks, nullptr);
    p->start = nullptr;
    if (hipEventCreateWithFlags(&p->start, hipEventDisableTiming) != hipSuccess) {
        p->start = nullptr;
        eq_pipeline_destroy(p);
        return EQ_EHIP;
    }
    for (uint32_t i = 0; i < n_blocks; ++i) {
        if (hipEventCreateWithFlags(&p->decoded[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->consumed[i], hipEventDisableTiming) != hipSuccess) {
            eq_pipeline_destroy(p);
            return EQ_EHIP;
        }
    }
    *out = p;
    return EQ_OK;
}

eq_status eq_pipeline_set_mode(eq_pipeline *p, uint32_t mode) {
    if (!p || (mode != EQ_PIPELINE_ALTERNATE && mode != EQ_PIPELINE_OVERLAP)) return EQ_EINVAL;
    p->overlap = mode;
    return EQ_OK;
}

eq_status eq_pipeline_run(eq_pipeline *p, const eq_block *blocks, uint32_t n_blocks,
                          uint16_t *d_buf0, uint16_t *d_buf1, const uint16_t *const *const *d_x,
                          float *const *const *d_y, void *decode_stream, void *gemv_stream) {
    if (!p || !blocks || !d_buf0 || !d_buf1 || !d_x || !d_y || n_blocks > p->n_blocks) return EQ_EINVAL;
    hipStream_t ds = static_cast<hipStream_t>(decode_stream);
    hipStream_t gs = static_cast<hipStream_t>(gemv_stream);
    uint16_t *buf[2] = {d_buf0, d_buf1};
    // the first two decodes overwrite buffers that GEMVs enqueued earlier on
    // gemv_stream (a previous run's last blocks) may still be reading
    if (hipEventRecord(p->start, gs) != hipSuccess || hipStreamWaitEvent(ds, p->start, 0) != hipSuccess)
        return EQ_EHIP;
    // the decode of block b waits for the GEMVs of block b - lag: b - 2 (the
    // last reader of its buffer) when it may run beside the GEMVs of b - 1,
    // b - 1 when the two streams take turns
    const uint32_t lag = p->overlap == EQ_PIPELINE_OVERLAP ? 2u : 1u;
    for (uint32_t b = 0; b < n_blocks; ++b) {
        uint16_t *dst = buf[b & 1u];
        if (b >= lag && hipStreamWaitEvent(ds, p->consumed[b - lag], 0) != hipSuccess) return EQ_EHIP;
        eq_status st = eq_decode_dequant_bf16(&blocks[b], dst, ds);
        if (st != EQ_OK) return st;
        if (hipEventRecord(p->decoded[b], ds) != hipSuccess) return EQ_EHIP;
        if (hipStreamWaitEvent(gs, p->decoded[b], 0) != hipSuccess) return EQ_EHIP;
        if (!d_x[b] || !d_y[b]) return EQ_EINVAL;
        for (uint32_t t = 0; t < blocks[b].n_tensors; ++t) {
            const eq_tensor_ref &r = blocks[b].tensors[t];
            st = eq_gemv_bf16(dst + r.out_offset, r.hdr.rows, r.hdr.cols, d_x[b][t], d_y[b][t], gs);
            if (st != EQ_OK) return st;
        }
        if (hipEventRecord(p->consumed[b], gs) != hipSuccess) return EQ_EHIP;
    }
    return EQ_OK;
}

eq_status eq_pipeline_destroy(eq_pipeline *p) {
    if (!p) return EQ_EINVAL;
    for (hipEvent_t e : p->decoded)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : p->consumed)
        if (e) (void)hipEventDestroy(e);
    if (p->start) (void)hipEventDestroy(p->start);
    delete p;
    return EQ_OK;
}

}  // extern "C"
