// Decode-round driver: one HIP graph per batch width.
//
// "Ignis" README, "The decode round": the round for all lanes is replayed
// from one captured graph per batch width (widths 1..8) rather than issued
// launch by launch.  Here a round is a list of weight matrices run in list
// order, each with its own activation input and output; the graph of width M
// holds one decode kernel per matrix (the verify-width kernel above 8 rows),
// one after the other on one stream, and nvfp4_round_run replays it.
//
// One kernel per matrix, not one launch for the round: on MI355X a graph's
// kernel boundary costs about 1.5 us, while telling every workgroup of the
// next matrix, on all eight XCDs, that the previous one is complete costs
// several device-scope round trips (about 6 us per matrix measured for a
// single-launch chain of plain reads with the round's byte sizes).
#include <new>
#include <vector>

#include "common.h"

struct nvfp4_round_plan {
    uint32_t magic;
    int max_M;
    std::vector<nvfp4_layer> layers;
    std::vector<nvfp4_gemm_plan*> plans;
    void* ws;
    size_t ws_bytes;
    size_t partial_off;  // shared offset of the partial sums (after every plan's counters)
    hipGraph_t graph[NVFP4_VERIFY_MAX_M];
    hipGraphExec_t exec[NVFP4_VERIFY_MAX_M];
    int nodes[NVFP4_VERIFY_MAX_M];
};

namespace nvfp4 {

static void free_round(nvfp4_round_plan* r) {
    for (int i = 0; i < NVFP4_VERIFY_MAX_M; ++i) {
        if (r->exec[i]) (void)hipGraphExecDestroy(r->exec[i]);
        if (r->graph[i]) (void)hipGraphDestroy(r->graph[i]);
    }
    for (nvfp4_gemm_plan* p : r->plans) nvfp4_gemm_destroy(p);
    r->magic = 0;
    delete r;
}

static int validate_layers(const nvfp4_layer* L, int n, int max_M) {
    if (!L) return set_error(NVFP4_EINVAL, "layers: NULL");
    if (n < 1) return set_error(NVFP4_EINVAL, "n_layers: %d < 1", n);
    if (max_M < 1 || max_M > NVFP4_VERIFY_MAX_M)
        return set_error(NVFP4_EINVAL, "max_M: %d outside [1, %d]", max_M, NVFP4_VERIFY_MAX_M);
    for (int i = 0; i < n; ++i) {
        const nvfp4_layer& l = L[i];
        if (l.K < 16 || l.K % 16) return set_error(NVFP4_EINVAL, "layers[%d].K: %d is not a positive multiple of 16", i, l.K);
        if (l.N < 1) return set_error(NVFP4_EINVAL, "layers[%d].N: %d < 1", i, l.N);
        if (!l.codes_dev || !l.scales_dev || !l.act_dev || !l.out_dev)
            return set_error(NVFP4_EINVAL, "layers[%d]: NULL buffer", i);
        if (((uintptr_t)l.codes_dev | (uintptr_t)l.scales_dev | (uintptr_t)l.act_dev) & 15)
            return set_error(NVFP4_EINVAL, "layers[%d]: codes/scales/act not 16-byte aligned", i);
        if ((uintptr_t)l.out_dev & 3) return set_error(NVFP4_EINVAL, "layers[%d].out: not 4-byte aligned", i);
        if (l.out_dtype != NVFP4_OUT_F32 && l.out_dtype != NVFP4_OUT_BF16)
            return set_error(NVFP4_EINVAL, "layers[%d].out_dtype: %d", i, l.out_dtype);
        if (l.act_op != NVFP4_ACT_INPUT && l.act_op != NVFP4_ACT_SWIGLU_PREV)
            return set_error(NVFP4_EINVAL, "layers[%d].act_op: %d", i, l.act_op);
        if (l.act_op == NVFP4_ACT_SWIGLU_PREV) {
            if (i == 0) return set_error(NVFP4_EINVAL, "layers[0].act_op: SWIGLU_PREV needs a previous matrix");
            if (L[i - 1].N != 2 * l.K)
                return set_error(NVFP4_EINVAL, "layers[%d].act_op: previous N = %d is not 2 K = %d", i,
                                 L[i - 1].N, 2 * l.K);
            if (L[i - 1].out_dtype != NVFP4_OUT_BF16)
                return set_error(NVFP4_EINVAL, "layers[%d].act_op: previous output is not bf16", i);
        }
    }
    return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

// Workspace of a per-matrix round: one counter region at the start, sized for
// the plan with the most counters, then one partial-sum region sized for the
// largest (decode or verify width).  The graph's nodes run one after another
// and each leaves its counters zeroed, so all of them share both regions.
static int round_layout(const nvfp4_layer* layers, int n_layers, int max_M, size_t* counters,
                        size_t* partials) {
    size_t mc = 0, mp = 0;
    for (int i = 0; i < n_layers; ++i) {
        nvfp4_gemm p;
        size_t b = 0;
        int st = nvfp4_gemm_create(&p, max_M, layers[i].K, layers[i].N, layers[i].out_dtype, &b);
        if (st) return st;
        if (p->dec.counter_bytes > mc) mc = p->dec.counter_bytes;
        if (p->dec.partial_bytes > mp) mp = p->dec.partial_bytes;
        if (p->ver.d.counter_bytes > mc) mc = p->ver.d.counter_bytes;
        if (p->ver.d.partial_bytes > mp) mp = p->ver.d.partial_bytes;
        nvfp4_gemm_destroy(p);
    }
    *counters = mc;
    *partials = mp;
    return NVFP4_OK;
}

int nvfp4_round_workspace_bytes(const nvfp4_layer* layers, int n_layers, int max_M,
                                size_t* workspace_bytes) {
    clear_error();
    int st = validate_layers(layers, n_layers, max_M);
    if (st) return st;
    if (!workspace_bytes) return set_error(NVFP4_EINVAL, "workspace_bytes: NULL");
    size_t c = 0, p = 0;
    st = round_layout(layers, n_layers, max_M, &c, &p);
    if (st) return st;
    *workspace_bytes = c + p;
    return NVFP4_OK;
}

int nvfp4_round_create(nvfp4_round* plan, const nvfp4_layer* layers, int n_layers, int max_M,
                       void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    if (!plan) return set_error(NVFP4_EINVAL, "plan: NULL");
    *plan = nullptr;
    int st = validate_layers(layers, n_layers, max_M);
    if (st) return st;
    size_t need_c = 0, need_p = 0;
    st = round_layout(layers, n_layers, max_M, &need_c, &need_p);
    if (st) return st;
    const size_t need = need_c + need_p;
    if (workspace_bytes < need)
        return set_error(NVFP4_EINVAL, "workspace_bytes: %zu < %zu needed", workspace_bytes, need);
    if (need && !workspace) return set_error(NVFP4_EINVAL, "workspace: NULL");
    if (workspace && ((uintptr_t)workspace & 15)) return set_error(NVFP4_EINVAL, "workspace: not 16-byte aligned");

    nvfp4_round_plan* r = new (std::nothrow) nvfp4_round_plan();
    if (!r) return set_error(NVFP4_EINVAL, "plan: out of host memory");
    r->magic = kRoundMagic;
    r->max_M = max_M;
    r->layers.assign(layers, layers + n_layers);
    r->ws = workspace;
    r->ws_bytes = workspace_bytes;
    r->partial_off = need_c;
    for (int i = 0; i < n_layers; ++i) {
        nvfp4_gemm p = nullptr;
        size_t b = 0;
        st = nvfp4_gemm_create(&p, max_M, layers[i].K, layers[i].N, layers[i].out_dtype, &b);
        if (st) {
            free_round(r);
            return st;
        }
        r->plans.push_back(p);
    }

    // Capture on a private non-blocking stream: the caller's stream may be the
    // null stream, which cannot be captured.
    hipStream_t user = (hipStream_t)stream;
    hipStream_t cap = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
    if (e != hipSuccess) {
        free_round(r);
        return hip_fail(e, "hipStreamCreateWithFlags");
    }
    st = NVFP4_OK;
    if (need) st = launch_fill_zero(workspace, need, user);
    if (!st) {
        e = hipStreamSynchronize(user);
        if (e != hipSuccess) st = hip_fail(e, "hipStreamSynchronize");
    }
    for (int M = 1; M <= max_M && !st; ++M) {
        e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) {
            st = hip_fail(e, "hipStreamBeginCapture");
            break;
        }
        int lst = NVFP4_OK;
        bool fused = false;  // the previous matrix's epilogue wrote this one's SwiGLU
        for (int i = 0; i < n_layers && !lst; ++i) {
            const nvfp4_layer& l = r->layers[i];
            if (l.act_op == NVFP4_ACT_SWIGLU_PREV && !fused)
                lst = launch_swiglu((const uint16_t*)r->layers[i - 1].out_dev,
                                    const_cast<uint16_t*>(l.act_dev), M, l.K, cap);
            if (lst) break;
            // A gate_up whose output feeds the next matrix through SwiGLU writes
            // that SwiGLU in its own epilogue where its plan allows, which saves
            // the SwiGLU kernel's launch.
            fused = i + 1 < n_layers && r->layers[i + 1].act_op == NVFP4_ACT_SWIGLU_PREV &&
                    decode_swiglu_fusable(r->plans[i], M);
            if (fused)
                lst = launch_decode_swiglu(r->plans[i], M, l.codes_dev, l.scales_dev,
                                           l.tensor_scale, l.act_dev, l.out_dev,
                                           const_cast<uint16_t*>(r->layers[i + 1].act_dev),
                                           workspace, r->partial_off, cap);
            else
                lst = run_gemm(r->plans[i], M, l.codes_dev, l.scales_dev, l.tensor_scale,
                               l.act_dev, l.out_dev, workspace,
                               RunOffsets{r->partial_off, 0, r->partial_off, 0, r->partial_off},
                               cap);
        }
        hipGraph_t g = nullptr;
        e = hipStreamEndCapture(cap, &g);
        if (lst) {
            if (g) (void)hipGraphDestroy(g);
            st = lst;
            break;
        }
        if (e != hipSuccess) {
            st = hip_fail(e, "hipStreamEndCapture");
            break;
        }
        r->graph[M - 1] = g;
        size_t nn = 0;
        if (hipGraphGetNodes(g, nullptr, &nn) == hipSuccess) r->nodes[M - 1] = (int)nn;
        e = hipGraphInstantiate(&r->exec[M - 1], g, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            st = hip_fail(e, "hipGraphInstantiate");
            break;
        }
        // Upload once so the first replay does not pay for it.
        e = hipGraphUpload(r->exec[M - 1], user);
        if (e != hipSuccess) {
            st = hip_fail(e, "hipGraphUpload");
            break;
        }
    }
    if (!st) {
        e = hipStreamSynchronize(user);
        if (e != hipSuccess) st = hip_fail(e, "hipStreamSynchronize");
    }
    (void)hipStreamDestroy(cap);
    if (st) {
        free_round(r);
        return st;
    }
    *plan = r;
    return NVFP4_OK;
}

int nvfp4_round_run(nvfp4_round plan, int M, void* stream) {
    clear_error();
    if (!plan || plan->magic != kRoundMagic) return set_error(NVFP4_ESTATE, "plan: invalid handle");
    if (M < 1 || M > plan->max_M) return set_error(NVFP4_EINVAL, "M: %d outside [1, max_M=%d]", M, plan->max_M);
    NVFP4_HIP(hipGraphLaunch(plan->exec[M - 1], (hipStream_t)stream));
    return NVFP4_OK;
}

int nvfp4_round_graph_nodes(nvfp4_round plan, int M) {
    if (!plan || plan->magic != kRoundMagic || M < 1 || M > plan->max_M) return 0;
    return plan->nodes[M - 1];
}

void nvfp4_round_destroy(nvfp4_round plan) {
    if (plan && plan->magic == kRoundMagic) free_round(plan);
}

}  // extern "C"
