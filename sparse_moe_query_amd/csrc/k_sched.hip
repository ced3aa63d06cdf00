// The attention schedule builder as a kernel of its own (one work group of 1024 threads): used
// when no router launch precedes the projection (the all-active GQA baseline).  Otherwise the
// router's first work group builds the schedule (k_router.hip).
#include "attn_sched_dev.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kLds = sched_dev::kHeader + 64 * 1024;

__global__ void __launch_bounds__(kThreads) attn_sched_kernel(SchedArgs a) {
    __shared__ __align__(16) unsigned char lds[kLds];
    attn_sched_block<kThreads>(a, lds, kLds);
}

}  // namespace

size_t attn_sched_scratch_bytes(const AttnCounts& ac) { return sched_array_bytes(ac.items, ac.tpl) + 64; }

SchedArgs make_sched_args(const GqeDims& D, const WorkPlan& P, char* ws) {
    const AttnCounts& ac = P.ac;
    SchedArgs a{};
    a.jobs = (AttnJob*)(ws + P.sched_jobs);
    a.merges = (AttnMerge*)(ws + P.sched_merges);
    a.gscratch = (int32_t*)(ws + P.sched_scratch);
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
    int nb = 1;
    while ((1 << nb) <= ac.maxlen) ++nb;
    a.nbits = nb;
    return a;
}

hipError_t launch_attn_sched(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st) {
    if (P.ac.njobs <= 0 || D.G > 64) return hipErrorInvalidValue;
    attn_sched_kernel<<<1, kThreads, 0, st>>>(make_sched_args(D, P, ws));
    return hipGetLastError();
}
