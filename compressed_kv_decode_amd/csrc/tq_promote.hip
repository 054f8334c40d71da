// k_promote: attention-weighted promotion with a sticky counter, one block
// per (sequence, kv head) of the batch (the body, with the passages of the
// pages it follows, is in tq_promote_body.h).
#include "tq_promote_body.h"

namespace tq {

template <int D, int CB>
__global__ __launch_bounds__(PNT) void k_promote(Dims dm, Ptrs P, LayerFmt F, int layer, CallSeqs cs) {
    promote_body<D, CB>(dm, P, F, layer, cs);
}

hipError_t launch_promote(const Dims& dm, const Ptrs& P, const LayerFmt& F, int layer, const CallSeqs& cs,
                          hipStream_t st) {
    if (cs.n == 0 || dm.ktop == 0) return hipSuccess;
    const int key = dm.d * 10 + F.cb;
    const dim3 grid(cs.n, dm.hkv);
    switch (key) {
        case 645: k_promote<64, 5><<<grid, PNT, 0, st>>>(dm, P, F, layer, cs); break;
        case 647: k_promote<64, 7><<<grid, PNT, 0, st>>>(dm, P, F, layer, cs); break;
        case 644: k_promote<64, 4><<<grid, PNT, 0, st>>>(dm, P, F, layer, cs); break;
        case 1285: k_promote<128, 5><<<grid, PNT, 0, st>>>(dm, P, F, layer, cs); break;
        case 1287: k_promote<128, 7><<<grid, PNT, 0, st>>>(dm, P, F, layer, cs); break;
        case 1284: k_promote<128, 4><<<grid, PNT, 0, st>>>(dm, P, F, layer, cs); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
