// check.hip - the optional debug validator, pkv_check_indices (gfx950).
//
// The store, dequant and decode calls take their device-resident index arrays (block table,
// context lengths, query-length prefix sums, slot mapping) as preconditions: reading them on the
// host would cost a synchronisation.  This kernel checks them on the device instead, for callers
// and tests that want to know before a call reads out of bounds:
//   * every context length lies in [0, max_blocks_per_seq * block_size];
//   * every block-table entry a sequence's context reaches (entries j < ceil(ctx / block_size))
//     names a block of the pool, [0, num_blocks); entries past the context are never read;
//   * cu_q_lens starts at 0 and never decreases, and each sequence's q_len is at most its
//     context length and at most the caller's max_q_len bound;
//   * every slot-mapping entry is below num_blocks * block_size (negative entries skip a token).
// One workgroup: the flags and the lowest offending indices gather in LDS (integer atomics), then
// are written whole, so the result needs no initial contents and no second launch.  Every read is
// inside the arrays' declared sizes, whatever their contents (a block-table row is walked for at
// most max_blocks_per_seq entries).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kNone = 0x7fffffff;

__global__ __launch_bounds__(kThreads) void check_kernel(CheckArgs a) {
    __shared__ int flags, first_seq, first_tok;
    if (threadIdx.x == 0) {
        flags = 0;
        first_seq = kNone;
        first_tok = kNone;
    }
    __syncthreads();
    int f = 0, fs = kNone, ft = kNone;
    const int64_t cap = (int64_t)a.mbs * a.bs;
    if (a.ctx) {
        for (int b = threadIdx.x; b < a.batch; b += kThreads) {
            const int ctx = a.ctx[b];
            int bad = 0;
            if (ctx < 0 || (a.mbs > 0 && ctx > cap)) bad |= kCheckContext;
            if (a.cu) {
                const int c0 = a.cu[b], c1 = a.cu[b + 1];
                if ((b == 0 && c0 != 0) || c1 < c0 || c1 - c0 > ctx || (a.max_q_len > 0 && c1 - c0 > a.max_q_len))
                    bad |= kCheckQlen;
            }
            if (bad) {
                f |= bad;
                fs = min(fs, b);
            }
        }
        if (a.bt) {
            const int64_t total = (int64_t)a.batch * a.mbs;
            for (int64_t i = threadIdx.x; i < total; i += kThreads) {
                const int b = (int)(i / a.mbs), j = (int)(i % a.mbs);
                const int ctx = a.ctx[b];
                if (ctx > 0 && (int64_t)j * a.bs < ctx) {  // the context reaches entry j
                    const int e = a.bt[i];
                    if (e < 0 || e >= a.num_blocks) {
                        f |= kCheckBlock;
                        fs = min(fs, b);
                    }
                }
            }
        }
    } else if (a.cu) {  // prefix sums alone (no context lengths to compare with)
        for (int b = threadIdx.x; b < a.batch; b += kThreads) {
            const int c0 = a.cu[b], c1 = a.cu[b + 1];
            if ((b == 0 && c0 != 0) || c1 < c0 || (a.max_q_len > 0 && c1 - c0 > a.max_q_len)) {
                f |= kCheckQlen;
                fs = min(fs, b);
            }
        }
    }
    if (a.slot) {
        const int64_t cap_s = (int64_t)a.num_blocks * a.bs;
        for (int t = threadIdx.x; t < a.num_tokens; t += kThreads)
            if (a.slot[t] >= cap_s) {
                f |= kCheckSlot;
                ft = min(ft, t);
            }
    }
    if (f) {
        atomicOr(&flags, f);
        if (fs != kNone) atomicMin(&first_seq, fs);
        if (ft != kNone) atomicMin(&first_tok, ft);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a.result[0] = flags;
        a.result[1] = first_seq == kNone ? -1 : first_seq;
        a.result[2] = first_tok == kNone ? -1 : first_tok;
        a.result[3] = 0;
    }
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
