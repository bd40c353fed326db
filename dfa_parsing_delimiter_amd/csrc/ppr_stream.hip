// Host streaming of inputs in partitions, with the transfer of one partition,
// the parse of the previous one and the return of the one before that
// overlapped on three HIP streams, two device buffers used in turn.
//
// Method: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw
// Data", the end-to-end streaming passage (double buffer, partitions whose
// transfer, parse and return overlap, Fig. 7). The pages hand the last
// incomplete record of a partition over to the next by copying its bytes in
// front of it (a carry-over region) and parsing them again. Here the parse
// itself is resumable: each partition starts in the DFA state where the
// previous one ended and inside its open field (PPR_PARSE_CONTINUE), and
// leaves its own open field to the next (PPR_PARSE_PARTIAL), so nothing is
// parsed twice and a record may span any number of partitions. The carried
// values are the end state, the open field's column and start, and the
// record and field counts so far; a small kernel turns each partition's
// 32-bit local results into 64-bit global ones.
#include <algorithm>
#include <vector>

#include <hip/hip_runtime.h>

#include "ppr.h"

namespace ppr {
namespace {

// partition-local fields -> global 64-bit ones. Field 0 of a partition ends
// the field that was open at its start: it starts where that field started
// (open_start) and is longer by the bytes before the partition.
__global__ void stream_rebase_kernel(const uint32_t* rec, const uint32_t* col, const uint32_t* off,
                                     const uint32_t* len, uint64_t nf, uint64_t rec_base, uint64_t part_base,
                                     uint64_t open_start, uint64_t* grec, uint32_t* gcol, uint64_t* goff, uint64_t* glen)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nf; i += (uint64_t)gridDim.x * blockDim.x) {
        grec[i] = rec_base + rec[i];
        gcol[i] = col[i];
        if (i == 0) {
            goff[i] = open_start;
            glen[i] = (uint64_t)len[i] + (part_base - open_start);
        } else {
            goff[i] = part_base + off[i];
            glen[i] = len[i];
        }
    }
}

struct DevBuf {
    uint8_t* in = nullptr;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    uint64_t cap = 0;  // field capacity of the arrays below
    uint32_t* f[4] = {nullptr, nullptr, nullptr, nullptr};
    uint64_t* grec = nullptr;
    uint32_t* gcol = nullptr;
    uint64_t* goff = nullptr;
    uint64_t* glen = nullptr;
    hipEvent_t in_done = nullptr, run_done = nullptr, out_done = nullptr;
};

void free_fields(DevBuf& b)
{
    for (auto& p : b.f) (void)hipFree(p), p = nullptr;
    (void)hipFree(b.grec);
    (void)hipFree(b.gcol);
    (void)hipFree(b.goff);
    (void)hipFree(b.glen);
    b.grec = nullptr;
    b.gcol = nullptr;
    b.goff = b.glen = nullptr;
    b.cap = 0;
}

bool alloc_fields(DevBuf& b, uint64_t cap)
{
    free_fields(b);
    cap = std::max<uint64_t>(cap, 1);
    bool ok = true;
    for (auto& p : b.f) ok = ok && hipMalloc((void**)&p, cap * 4) == hipSuccess;
    ok = ok && hipMalloc((void**)&b.grec, cap * 8) == hipSuccess;
    ok = ok && hipMalloc((void**)&b.gcol, cap * 4) == hipSuccess;
    ok = ok && hipMalloc((void**)&b.goff, cap * 8) == hipSuccess;
    ok = ok && hipMalloc((void**)&b.glen, cap * 8) == hipSuccess;
    if (ok) b.cap = cap;
    return ok;
}

}  // namespace
}  // namespace ppr

using namespace ppr;

extern "C" int ppr_parse_stream(const uint8_t* h_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                                ppr_stream_out_t* out, uint64_t partition_bytes, const ppr_parse_opts_t* opts)
{
    if (!out || !dfa || !class_map || (n && !h_bytes)) return PPR_EINVAL;
    if (partition_bytes == 0 || partition_bytes > 0xffff0000ull) return PPR_EINVAL;
    if (opts && (opts->flags || opts->start_state || opts->start_column)) return PPR_EINVAL;
    if (out->cap_fields && (!out->record_idx || !out->column_ids || !out->field_offsets || !out->field_lengths))
        return PPR_EINVAL;
    ppr_parse_opts_t o{};
    if (opts) {
        o.chunk_bytes = opts->chunk_bytes;
        o.path = opts->path;
        o.expected_columns = opts->expected_columns;
    }
    const uint64_t pb = std::min<uint64_t>(partition_bytes, std::max<uint64_t>(n, 1));
    const uint64_t parts = n ? (n + pb - 1) / pb : 1;
    const size_t wsb = ppr_parse_workspace_bytes(pb, &o);
    if (!wsb) return PPR_EINVAL;

    hipStream_t s_in = nullptr, s_run = nullptr, s_out = nullptr;
    DevBuf buf[2];
    int rc = PPR_OK;
    auto hip_ok = [&](hipError_t e) {
        if (e != hipSuccess && rc == PPR_OK) rc = PPR_EHIP;
        return e == hipSuccess;
    };
    // (default priority streams; every wait between them is an event)
    bool ok = hip_ok(hipStreamCreateWithFlags(&s_in, hipStreamNonBlocking)) &&
              hip_ok(hipStreamCreateWithFlags(&s_run, hipStreamNonBlocking)) &&
              hip_ok(hipStreamCreateWithFlags(&s_out, hipStreamNonBlocking));
    for (auto& b : buf) {
        ok = ok && hip_ok(hipMalloc((void**)&b.in, pb)) && hip_ok(hipMalloc(&b.ws, wsb)) &&
             hip_ok(hipMemsetAsync(b.ws, 0, wsb, s_run)) &&
             hip_ok(hipEventCreateWithFlags(&b.in_done, hipEventDisableTiming)) &&
             hip_ok(hipEventCreateWithFlags(&b.run_done, hipEventDisableTiming)) &&
             hip_ok(hipEventCreateWithFlags(&b.out_done, hipEventDisableTiming));
        b.ws_bytes = wsb;
        ok = ok && (alloc_fields(b, std::min<uint64_t>(pb + 1, pb / 4 + 4096)) || (rc = PPR_EHIP, false));
    }

    // carried from partition to partition
    uint32_t state = dfa->start_state, col = 0;
    uint64_t open_start = 0, rec_base = 0, field_base = 0, bad = 0;
    int64_t err = -1, first_bad = -1;
    uint32_t cmin = 0xffffffffu, cmax = 0;
    auto len_of = [&](uint64_t k) { return k * pb >= n ? 0 : std::min<uint64_t>(pb, n - k * pb); };
    auto send = [&](uint64_t k) {  // transfer of partition k, once the parse two partitions back has released its buffer
        DevBuf& b = buf[k & 1];
        if (k >= 2) hip_ok(hipStreamWaitEvent(s_in, buf[k & 1].run_done, 0));
        if (len_of(k)) hip_ok(hipMemcpyAsync(b.in, h_bytes + k * pb, len_of(k), hipMemcpyHostToDevice, s_in));
        hip_ok(hipEventRecord(b.in_done, s_in));
    };
    if (ok) send(0);
    for (uint64_t k = 0; ok && k < parts; ++k) {
        DevBuf& b = buf[k & 1];
        const uint64_t len = len_of(k), part_base = k * pb;
        if (k + 1 < parts) send(k + 1);
        hip_ok(hipStreamWaitEvent(s_run, b.in_done, 0));
        if (k >= 2) hip_ok(hipStreamWaitEvent(s_run, b.out_done, 0));  // its 64-bit arrays are free again
        ppr_parse_opts_t ok_opts = o;
        ok_opts.flags = (k ? PPR_PARSE_CONTINUE : 0u) | (k + 1 < parts ? PPR_PARSE_PARTIAL : 0u);
        ok_opts.start_state = k ? state : 0u;
        ok_opts.start_column = k ? col : 0u;
        ppr_parse_out_t po{};
        int prc = PPR_OK;
        for (int attempt = 0; attempt < 2; ++attempt) {  // size, then fill
            po = ppr_parse_out_t{};
            po.record_idx = b.f[0];
            po.column_ids = b.f[1];
            po.field_offsets = b.f[2];
            po.field_lengths = b.f[3];
            po.cap_fields = b.cap;
            prc = ppr_parse_async(b.in, len, dfa, class_map, &po, b.ws, b.ws_bytes, &ok_opts, s_run);
            if (prc == PPR_OK) prc = ppr_parse_results(b.ws, len, &po, s_run);
            if (prc != PPR_ECAPACITY) break;
            // (a return still reading this buffer's arrays must end before they are replaced)
            hip_ok(hipStreamSynchronize(s_out));
            if (!alloc_fields(b, po.n_fields + po.n_fields / 8 + 1024)) prc = PPR_EHIP;
        }
        if (prc != PPR_OK) {
            rc = prc;
            break;
        }
        const uint64_t nf = po.n_fields;
        if (nf) {
            const uint32_t grid = (uint32_t)std::min<uint64_t>((nf + 255) / 256, 8192);
            hipLaunchKernelGGL(stream_rebase_kernel, dim3(grid), dim3(256), 0, s_run, b.f[0], b.f[1], b.f[2], b.f[3],
                               nf, rec_base, part_base, open_start, b.grec, b.gcol, b.goff, b.glen);
            hip_ok(hipGetLastError());
        }
        hip_ok(hipEventRecord(b.run_done, s_run));
        // the return of this partition's fields (those within the caller's capacity)
        hip_ok(hipStreamWaitEvent(s_out, b.run_done, 0));
        const uint64_t room = field_base < out->cap_fields ? std::min<uint64_t>(nf, out->cap_fields - field_base) : 0;
        if (room) {
            hip_ok(hipMemcpyAsync(out->record_idx + field_base, b.grec, room * 8, hipMemcpyDeviceToHost, s_out));
            hip_ok(hipMemcpyAsync(out->column_ids + field_base, b.gcol, room * 4, hipMemcpyDeviceToHost, s_out));
            hip_ok(hipMemcpyAsync(out->field_offsets + field_base, b.goff, room * 8, hipMemcpyDeviceToHost, s_out));
            hip_ok(hipMemcpyAsync(out->field_lengths + field_base, b.glen, room * 8, hipMemcpyDeviceToHost, s_out));
        }
        hip_ok(hipEventRecord(b.out_done, s_out));
        // carry to the next partition
        if (err < 0 && po.error_pos >= 0) err = (int64_t)part_base + po.error_pos;
        if (first_bad < 0 && po.first_bad_record >= 0) first_bad = (int64_t)rec_base + po.first_bad_record;
        bad += po.bad_records;
        if (po.n_records) {
            cmin = std::min(cmin, po.min_columns);
            cmax = std::max(cmax, po.max_columns);
        }
        if (nf) open_start = part_base + po.tail_start;  // (no terminator: the open field goes on)
        rec_base += po.n_records;
        field_base += nf;
        state = po.end_state;
        col = po.tail_column;
    }
    hip_ok(hipStreamSynchronize(s_out));
    hip_ok(hipStreamSynchronize(s_run));
    hip_ok(hipStreamSynchronize(s_in));
    for (auto& b : buf) {
        free_fields(b);
        (void)hipFree(b.in);
        (void)hipFree(b.ws);
        if (b.in_done) (void)hipEventDestroy(b.in_done);
        if (b.run_done) (void)hipEventDestroy(b.run_done);
        if (b.out_done) (void)hipEventDestroy(b.out_done);
    }
    if (s_in) (void)hipStreamDestroy(s_in);
    if (s_run) (void)hipStreamDestroy(s_run);
    if (s_out) (void)hipStreamDestroy(s_out);
    out->n_fields = field_base;
    out->n_records = rec_base;
    out->error_pos = err;
    out->end_state = state;
    out->min_columns = cmin == 0xffffffffu ? 0u : cmin;
    out->max_columns = cmax;
    out->partitions = (uint32_t)parts;
    out->bad_records = bad;
    out->first_bad_record = first_bad;
    if (rc != PPR_OK) return rc;
    return field_base > out->cap_fields ? PPR_ECAPACITY : PPR_OK;
}
