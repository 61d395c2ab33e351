// The whole sparse forward in four launches (rec_sparse_din_fwd).  The deep
// and the sequence side each need a sums pass and then a pass that consumes
// the sums; the two sides are independent, so each pair runs as one launch
// whose blocks split by index between the two kinds of work:
//   1. KJT block/chunk sums | plan block/chunk sums;
//   2. plan build (positions, entries, rows, group starts) | embedding bags
//      with offsets derived in the bags;
//   3. DIN attention (rec_din.hip).
// Every kernel on the path costs a fixed ~2 us inside a graph whatever its
// size, so two fewer launches save about as much as the first pass costs.
#include "rec_embbag_dev.h"
#include "rec_scan_dev.h"

namespace rec {
namespace {

struct FwdSums {
    const int32_t* lengths;     // deep [T][B]
    const int32_t* seq_lengths;
    int64_t B, nK, G;
    int64_t* bs;
    int64_t* segp;
    int64_t* chp;
    int64_t* plan_sums;
    int32_t* hdr;
    int64_t nkjt;               // blocks of KJT sums (the rest are plan sums)
    int32_t max_len;
};

__global__ __launch_bounds__(kScanThreads) void k_fwd_sums(const FwdSums a) {
    if ((int64_t)blockIdx.x < a.nkjt)
        k_kjt_sums_body(a.lengths, a.B, a.nK, a.G, a.bs, a.segp, a.chp, blockIdx.x);
    else
        k_plan_sums_body(a.seq_lengths, a.B, a.max_len, a.plan_sums, a.hdr, blockIdx.x - a.nkjt);
}

template <bool kHashSeq, bool kHashEmb>
__global__ __launch_bounds__(256) void k_fwd_gather(const PlanArgs p, const EmbArgs e, int64_t nbuild) {
    if ((int64_t)blockIdx.x < nbuild)
        k_plan_build_body<kHashSeq>(p, blockIdx.x, nbuild);
    else
        k_embbag_fwd_body<kHashEmb, true>(e, blockIdx.x - nbuild);
}

}  // namespace

hipError_t launch_fwd_front(const PlanArgs& p, const EmbArgs& e, hipStream_t s) {
    const PlanLayout L = plan_layout(p.B, p.max_len);
    const KjtLayout k = kjt_layout(e.T, e.B);
    char* pl = (char*)p.plan;
    FwdSums a;
    a.lengths = e.lengths;
    a.seq_lengths = p.seq_lengths;
    a.B = p.B;
    a.nK = k.nK;
    a.G = k.G;
    a.bs = (int64_t*)e.kjt_bs;
    a.segp = (int64_t*)e.kjt_segp;
    a.chp = (int64_t*)e.kjt_chp;
    a.plan_sums = (int64_t*)(pl + L.off_sums);
    a.hdr = (int32_t*)pl;
    a.nkjt = (int64_t)e.T * k.nK;
    a.max_len = p.max_len;
    REC_LAUNCH(REC_TIME_SUMS, k_fwd_sums, dim3((unsigned)(a.nkjt + L.nblocks)), dim3(kScanThreads), 0, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t nbuild = (p.B + kPlanChunk - 1) / kPlanChunk;
    const int64_t emb_blocks = ((int64_t)((e.T + 1) / 2) * ((e.B + 31) / 32) + kWaves - 1) / kWaves;
    const bool hs = p.tab[0].kind == REC_HASH || p.tab[1].kind == REC_HASH || p.tab[2].kind == REC_HASH;
    bool he = false;
    for (int t = 0; t < e.T; ++t) he = he || e.tab[t].kind == REC_HASH;
    const dim3 grid((unsigned)(nbuild + emb_blocks)), block(256);
    if (hs && he) REC_LAUNCH(REC_TIME_GATHER, (k_fwd_gather<true, true>), grid, block, 0, s, p, e, nbuild);
    else if (hs) REC_LAUNCH(REC_TIME_GATHER, (k_fwd_gather<true, false>), grid, block, 0, s, p, e, nbuild);
    else if (he) REC_LAUNCH(REC_TIME_GATHER, (k_fwd_gather<false, true>), grid, block, 0, s, p, e, nbuild);
    else REC_LAUNCH(REC_TIME_GATHER, (k_fwd_gather<false, false>), grid, block, 0, s, p, e, nbuild);
    return hipGetLastError();
}

}  // namespace rec
