// The attention schedule builder as a kernel of its own (one work group of 1024 threads): used
// when no router launch precedes the projection (the all-active GQA baseline).  Otherwise the
// router's first work group builds the schedule (k_router.hip).
#include "attn_sched_dev.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kLds = sched_dev::kHeader + 8 * 8192;

__global__ void __launch_bounds__(kThreads) attn_sched_kernel(SchedArgs a) {
    __shared__ __align__(16) unsigned char lds[kLds];
    attn_sched_block<kThreads>(a, lds, kLds);
}

}  // namespace

size_t attn_sched_scratch_bytes(const AttnCounts& ac) {
    return (size_t)(3 * (ac.items + 1) + 2 * ac.tpl) * 4 + 64 + (size_t)sched_npow2(ac.tpl) * 8;
}

SchedArgs make_sched_args(const GqeDims& D, const WorkPlan& P, char* ws) {
    const AttnCounts& ac = P.ac;
    SchedArgs a{};
    a.jobs = (AttnJob*)(ws + P.sched_jobs);
    a.merges = (AttnMerge*)(ws + P.sched_merges);
    int32_t* sc = (int32_t*)(ws + P.sched_scratch);
    a.tstart = sc;
    a.sstart = a.tstart + (ac.items + 1);
    a.mstart = a.sstart + (ac.items + 1);
    a.tf = a.mstart + (ac.items + 1);
    a.rank = a.tf + ac.tpl;
    // 8-byte aligned keys after the int32 arrays
    const size_t koff = ((size_t)(3 * (ac.items + 1) + 2 * ac.tpl) * 4 + 63) & ~(size_t)63;
    a.gkeys = (uint64_t*)(ws + P.sched_scratch + koff);
    a.B = P.B;
    a.S = P.S;
    a.G = D.G;
    a.k = D.k;
    a.s = D.s;
    a.skv = D.skv;
    a.C = ac.chunk;
    a.items = ac.items;
    a.tpl = ac.tpl;
    a.maxlen = ac.maxlen;
    a.npow2 = sched_npow2(ac.tpl);
    return a;
}

hipError_t launch_attn_sched(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st) {
    if (P.ac.njobs <= 0 || D.G > 64) return hipErrorInvalidValue;
    attn_sched_kernel<<<1, kThreads, 0, st>>>(make_sched_args(D, P, ws));
    return hipGetLastError();
}
