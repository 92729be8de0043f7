// The C ABI's host-side validation and workspace arithmetic, built with the
// host sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) together
// with the whole library.  Every call here is refused by validation, is a
// documented no-op, or is a size query: nothing reaches a kernel, so it runs
// without a GPU.  Pointers are fake device addresses, never dereferenced.
// Exit status 0 = every expectation held and no sanitizer report.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda.h"
#include "kda_internal.hpp"

namespace {

int failures = 0;

void expect(int line, kda_status got, kda_status want)
{
    if (got != want) {
        std::fprintf(stderr, "line %d: status %d (%s), expected %d\n", line, int(got),
                     kda_status_str(got), int(want));
        ++failures;
    }
}
#define EXPECT(call, want) expect(__LINE__, (call), (want))

void* const P = reinterpret_cast<void*>(0x10000);     // 16-byte aligned
void* const MIS = reinterpret_cast<void*>(0x10008);   // 8-byte aligned only
void* const W = reinterpret_cast<void*>(0x20000);     // 256-byte aligned
const float* const PF = static_cast<const float*>(P);
float* const OF = static_cast<float*>(P);
const int32_t* const CU = static_cast<const int32_t*>(P);
const kda_dtype BF = KDA_BF16;

kda_status prefill(const void* q, const void* k, const float* s1ok, int64_t B, int64_t T, int64_t H,
                   int64_t dk, kda_dtype dt, void* ws = nullptr, int64_t wb = 0)
{
    return kda_prefill(q, k, P, P, PF, nullptr, OF, const_cast<float*>(s1ok), B, T, H, dk, 128, dt,
                       ws, wb, nullptr);
}

void prefill_checks()
{
    EXPECT(prefill(nullptr, P, PF, 1, 4, 2, 128, BF), KDA_ERR_NULL);
    EXPECT(prefill(P, MIS, PF, 1, 4, 2, 128, BF), KDA_ERR_ALIGN);
    EXPECT(prefill(P, P, static_cast<const float*>(MIS), 1, 4, 2, 128, BF), KDA_ERR_ALIGN);
    EXPECT(prefill(P, P, PF, 1, 4, 2, 64, BF), KDA_ERR_UNSUPPORTED);
    EXPECT(prefill(P, P, PF, 1, 4, 0, 128, BF), KDA_ERR_SHAPE);
    EXPECT(prefill(P, P, PF, 1, 1, 65537, 128, BF), KDA_ERR_SHAPE);
    EXPECT(prefill(P, P, PF, -1, 4, 2, 128, BF), KDA_ERR_SHAPE);
    EXPECT(prefill(P, P, PF, 1, int64_t(1) << 40, 2, 128, BF), KDA_ERR_SHAPE);
    EXPECT(prefill(P, P, PF, INT64_MAX, INT64_MAX, 65536, 128, BF), KDA_ERR_SHAPE);
    EXPECT(prefill(P, P, PF, 1, 4, 2, 128, kda_dtype(2)), KDA_ERR_DTYPE);
    EXPECT(kda_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4,
                       2, 128, 128, BF, nullptr, 0, nullptr),
           KDA_OK);
    EXPECT(kda_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0,
                       2, 128, 128, BF, nullptr, 0, nullptr),
           KDA_OK);
    // workspace rules
    EXPECT(prefill(P, P, PF, 1, 4, 2, 128, BF, nullptr, 4096), KDA_ERR_NULL);
    EXPECT(prefill(P, P, PF, 1, 4, 2, 128, BF, static_cast<char*>(P) + 16, 4096), KDA_ERR_ALIGN);
    EXPECT(prefill(P, P, PF, 1, 4, 2, 128, BF, W, KDA_WORKSPACE_AUTO), KDA_ERR_WORKSPACE);
    EXPECT(prefill(P, P, PF, 1, 4, 2, 128, BF, nullptr, -2), KDA_ERR_WORKSPACE);
    EXPECT(kda_prefill_noalloc(nullptr, P, P, P, PF, nullptr, OF, OF, 1, 4, 2, 128, 128, BF, nullptr),
           KDA_ERR_NULL);
    EXPECT(kda_prefill_noalloc(P, P, P, P, PF, nullptr, OF, OF, 1, int64_t(1) << 40, 2, 128, 128, BF,
                               nullptr),
           KDA_ERR_SHAPE);
    EXPECT(kda_prefill_raw(P, P, P, P, PF, nullptr, OF, OF, 1, 4, 2, 96, 128, BF, nullptr, 0, nullptr),
           KDA_ERR_UNSUPPORTED);
}

void varlen_checks()
{
    auto call = [](const int32_t* cu, int64_t N, int64_t Tt, int64_t H, kda_dtype dt) {
        return kda_varlen_prefill(P, P, P, P, PF, cu, N, Tt, nullptr, OF, OF, H, 128, 128, dt,
                                  nullptr, 0, nullptr);
    };
    EXPECT(call(nullptr, 2, 8, 2, BF), KDA_ERR_NULL);
    EXPECT(call(reinterpret_cast<const int32_t*>(0x10004), 2, 8, 2, BF), KDA_ERR_ALIGN);
    EXPECT(call(CU, -1, 8, 2, BF), KDA_ERR_SHAPE);
    EXPECT(call(CU, 2, int64_t(1) << 31, 2, BF), KDA_ERR_SHAPE);
    EXPECT(call(CU, INT64_MAX, 8, 2, BF), KDA_ERR_SHAPE);
    EXPECT(call(CU, 2, 8, 65537, BF), KDA_ERR_SHAPE);
    EXPECT(call(CU, 2, 8, 2, kda_dtype(7)), KDA_ERR_DTYPE);
    EXPECT(kda_varlen_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 8, nullptr,
                              nullptr, nullptr, 2, 128, 128, BF, nullptr, 0, nullptr),
           KDA_OK);
    EXPECT(kda_varlen_prefill_raw(P, P, P, P, PF, CU, 2, 8, nullptr, OF, OF, 0, 128, 128, BF,
                                  nullptr, 0, nullptr),
           KDA_ERR_SHAPE);
    EXPECT(kda_varlen_prefill_slots(P, P, P, P, PF, CU, 2, 8, OF, CU, CU, -2, OF, 2, 128, 128, BF,
                                    nullptr, 0, nullptr),
           KDA_ERR_SHAPE);
    EXPECT(kda_varlen_prefill_slots(P, P, P, P, PF, CU, 2, 8, nullptr, CU, CU, 4, OF, 2, 128, 128,
                                    BF, nullptr, 0, nullptr),
           KDA_ERR_NULL);
}

void decode_checks()
{
    EXPECT(kda_decode_step(nullptr, P, P, P, PF, OF, OF, 2, 2, 128, 128, BF, nullptr), KDA_ERR_NULL);
    EXPECT(kda_decode_step(P, P, P, P, PF, static_cast<float*>(MIS), OF, 2, 2, 128, 128, BF, nullptr),
           KDA_ERR_ALIGN);
    EXPECT(kda_decode_step(P, P, P, P, PF, OF, OF, -3, 2, 128, 128, BF, nullptr), KDA_ERR_SHAPE);
    EXPECT(kda_decode_step(P, P, P, P, PF, OF, OF, INT64_MAX, 65536, 128, 128, BF, nullptr),
           KDA_ERR_SHAPE);
    EXPECT(kda_decode_step(P, P, P, P, PF, OF, OF, 2, 2, 127, 128, BF, nullptr), KDA_ERR_UNSUPPORTED);
    EXPECT(kda_decode_step(P, P, P, P, PF, OF, OF, 2, 2, 128, 128, kda_dtype(3), nullptr),
           KDA_ERR_DTYPE);
    EXPECT(kda_decode_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 2, 128,
                           128, BF, nullptr),
           KDA_OK);
    EXPECT(kda_decode_step_raw(P, P, P, P, PF, OF, OF, 2, 0, 128, 128, BF, nullptr), KDA_ERR_SHAPE);
    EXPECT(kda_decode_tokens(P, P, P, P, PF, OF, nullptr, OF, 2, 17, 2, 128, 128, BF, nullptr),
           KDA_ERR_SHAPE);
    EXPECT(kda_decode_tokens(P, P, P, P, PF, OF, nullptr, OF, 2, 0, 2, 128, 128, BF, nullptr),
           KDA_ERR_SHAPE);
    EXPECT(kda_decode_tokens(P, P, P, P, PF, OF, reinterpret_cast<const int32_t*>(MIS), OF, 2, 4, 2,
                             128, 128, BF, nullptr),
           KDA_ERR_ALIGN);
    EXPECT(kda_decode_step_slots(P, P, P, P, PF, OF, CU, int64_t(1) << 40, OF, 2, 2, 128, 128, BF,
                                 nullptr),
           KDA_ERR_SHAPE);
    EXPECT(kda_decode_step_slots(P, P, P, P, PF, OF, nullptr, 4, OF, 2, 2, 128, 128, BF, nullptr),
           KDA_ERR_NULL);
}

void backward_checks()
{
    auto call = [](const void* q, const float* ds0, int64_t B, int64_t T, int64_t H, int64_t dk,
                   kda_dtype dt, void* ws, int64_t wb) {
        return kda_backward(q, P, P, P, PF, nullptr, PF, nullptr, OF, OF, OF, OF, OF,
                            const_cast<float*>(ds0), B, T, H, dk, 128, dt, ws, wb, nullptr);
    };
    EXPECT(call(nullptr, PF, 1, 4, 2, 128, BF, nullptr, 0), KDA_ERR_NULL);
    EXPECT(call(MIS, PF, 1, 4, 2, 128, BF, nullptr, 0), KDA_ERR_ALIGN);
    EXPECT(call(P, static_cast<const float*>(MIS), 1, 4, 2, 128, BF, nullptr, 0), KDA_ERR_ALIGN);
    EXPECT(call(P, PF, -1, 4, 2, 128, BF, nullptr, 0), KDA_ERR_SHAPE);
    EXPECT(call(P, PF, 1, int64_t(1) << 40, 2, 128, BF, nullptr, 0), KDA_ERR_SHAPE);
    EXPECT(call(P, PF, INT64_MAX, INT64_MAX, 2, 128, BF, nullptr, 0), KDA_ERR_SHAPE);
    EXPECT(call(P, PF, 1, 4, 65537, 128, BF, nullptr, 0), KDA_ERR_SHAPE);
    EXPECT(call(P, PF, 1, 4, 2, 64, BF, nullptr, 0), KDA_ERR_UNSUPPORTED);
    EXPECT(call(P, PF, 1, 4, 2, 128, kda_dtype(2), nullptr, 0), KDA_ERR_DTYPE);
    EXPECT(call(P, PF, 1, 4, 2, 128, BF, W, KDA_WORKSPACE_AUTO), KDA_ERR_WORKSPACE);
    EXPECT(call(P, PF, 1, 4, 2, 128, BF, W, -5), KDA_ERR_WORKSPACE);
    EXPECT(kda_backward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 2, 128, 128, BF,
                        nullptr, 0, nullptr),
           KDA_OK);
    EXPECT(kda_varlen_backward(P, P, P, P, PF, nullptr, 2, 8, nullptr, PF, nullptr, OF, OF, OF, OF,
                               OF, OF, 2, 128, 128, BF, nullptr, 0, nullptr),
           KDA_ERR_NULL);
    EXPECT(kda_varlen_backward(P, P, P, P, PF, CU, 2, int64_t(1) << 31, nullptr, PF, nullptr, OF, OF,
                               OF, OF, OF, OF, 2, 128, 128, BF, nullptr, 0, nullptr),
           KDA_ERR_SHAPE);
}

bool have_device = false;

// Size queries: refusals leave 0; accepted sizes are non-negative and, for the
// backward, grow with the problem; nothing overflows on the largest shapes.
// The bf16 prefill sizes need the device's compute units: without a device
// those queries return KDA_ERR_HIP.
void size_checks()
{
    int64_t b = -7;
    EXPECT(kda_prefill_workspace_size(1, 4, 0, 128, 128, BF, KDA_PLAN_FULL, &b), KDA_ERR_SHAPE);
    if (b != 0) ++failures;
    EXPECT(kda_prefill_workspace_size(1, 4, 2, 128, 128, BF, kda_plan(3), &b), KDA_ERR_SHAPE);
    EXPECT(kda_prefill_workspace_size(1, 4, 2, 128, 128, BF, KDA_PLAN_FULL, nullptr), KDA_ERR_NULL);
    EXPECT(kda_backward_workspace_size(INT64_MAX, INT64_MAX, 65536, 128, 128, BF, &b), KDA_ERR_SHAPE);
    if (b != 0) ++failures;
    const kda_plan plans[3] = {KDA_PLAN_FULL, KDA_PLAN_SEGMENTS, KDA_PLAN_UNSEGMENTED};
    const int64_t shapes[][3] = {{1, 1 << 20, 32}, {8, 4096, 32}, {64, 1, 32}, {1, 65, 65536},
                                 {4096, 8192, 1}, {1, (int64_t(1) << 31) - 1, 1}};
    for (const auto& s : shapes) {
        for (kda_plan p : plans) {
            int64_t d = -1, v = -1;
            const kda_status sd = kda_prefill_workspace_size(s[0], s[1], s[2], 128, 128, BF, p, &d);
            const int64_t tt = s[0] * s[1] < (int64_t(1) << 31) ? s[0] * s[1] : 1;
            const kda_status sv = kda_varlen_prefill_workspace_size(s[0], tt, s[2], 128, 128, BF, p, &v);
            if (have_device) {
                EXPECT(sd, KDA_OK);
                EXPECT(sv, KDA_OK);
            } else if ((sd != KDA_OK && sd != KDA_ERR_HIP) || (sv != KDA_OK && sv != KDA_ERR_HIP)) {
                ++failures;
            }
            if (d < 0 || v < 0) ++failures;
        }
        int64_t b16 = -1, b32 = -1;
        EXPECT(kda_backward_workspace_size(s[0], s[1], s[2], 128, 128, BF, &b16), KDA_OK);
        EXPECT(kda_backward_workspace_size(s[0], s[1], s[2], 128, 128, KDA_F32, &b32), KDA_OK);
        if (b16 <= 0 || b32 <= 0) ++failures;
    }
    int64_t small = 0, big = 0;
    EXPECT(kda_backward_workspace_size(1, 4096, 32, 128, 128, BF, &small), KDA_OK);
    EXPECT(kda_backward_workspace_size(1, 1 << 20, 32, 128, 128, BF, &big), KDA_OK);
    if (!(big > small)) ++failures;
    EXPECT(kda_set_prefill_segment(100), KDA_ERR_SHAPE);
    EXPECT(kda_set_prefill_segment(-64), KDA_ERR_SHAPE);
    EXPECT(kda_set_prefill_segment(64), KDA_OK);
    for (const auto& s : shapes) {  // the shortest forced segment: the most slots
        int64_t d = -1;
        const kda_status sd = kda_prefill_workspace_size(s[0], s[1], s[2], 128, 128, BF, KDA_PLAN_FULL, &d);
        if (sd != KDA_OK && !(sd == KDA_ERR_HIP && !have_device)) ++failures;
    }
    EXPECT(kda_set_prefill_segment(0), KDA_OK);
}

// The plans themselves, on 256 and on 1 compute units: segments cover every
// token, are whole chunks, and the workspace holds every slot.
void plan_checks()
{
    const int64_t dense[][3] = {{1, 1 << 20, 32}, {8, 4096, 32}, {64, 1, 32}, {1, 65, 65536},
                                {2, 3500, 2}, {4096, 8192, 1}, {1, (int64_t(1) << 31) - 1, 1}};
    const int64_t forced[] = {0, 64, 1024, 4096};
    for (int n_cu : {256, 1}) {
        for (const auto& s : dense) {
            for (int64_t f : forced) {
                for (int tier = 0; tier < 3; ++tier) {
                    const kda::PrefillPlan p = kda::plan_prefill_scan(false, s[0], s[1], s[0] * s[1], s[2],
                                                                      n_cu, f, tier);
                    if (!p.segmented) continue;
                    const bool ok = p.seg > 0 && p.seg % kda::kChunk == 0 && p.seg0 > 0 &&
                                    p.seg0 <= p.seg && p.nseg_dense >= 2 &&
                                    p.seg0 + (p.nseg_dense - 1) * p.seg >= s[1] &&
                                    p.seg0 + (p.nseg_dense - 2) * p.seg < s[1] &&
                                    p.slots == s[0] * p.nseg_dense &&
                                    p.ws_bytes >= static_cast<size_t>(p.slots) * s[2] * 3 *
                                                      kda::kStateFloats * sizeof(float);
                    if (!ok) {
                        std::fprintf(stderr, "dense plan %lld x %lld x %lld, forced %lld, tier %d\n",
                                     (long long)s[0], (long long)s[1], (long long)s[2], (long long)f, tier);
                        ++failures;
                    }
                }
                const kda::PrefillPlan q = kda::plan_prefill_scan(true, s[0], 0, s[0] * s[1], s[2], n_cu, f, 1);
                if (q.segmented && (q.slots > q.n_segs || q.seg_min > q.seg || q.seg_min % kda::kChunk)) {
                    std::fprintf(stderr, "packed plan %lld x %lld\n", (long long)s[0], (long long)s[1]);
                    ++failures;
                }
            }
            const kda::BackwardPlan b = kda::plan_backward(false, s[0], s[1], 0, s[2], true);
            if (!b.chunked || b.n_ids < s[0] * s[1] / kda::kChunk + 1) ++failures;
        }
    }
}

}  // namespace

int main()
{
    int n_dev = 0;
    have_device = hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0;
    (void)hipGetLastError();  // no device is not an error here

    if (kda_abi_version() != KDA_ABI_VERSION) ++failures;
    for (int s = -1; s < 12; ++s)
        if (!kda_status_str(kda_status(s)) || !std::strlen(kda_status_str(kda_status(s)))) ++failures;
    prefill_checks();
    varlen_checks();
    decode_checks();
    backward_checks();
    size_checks();
    plan_checks();
    std::printf("abi driver: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
