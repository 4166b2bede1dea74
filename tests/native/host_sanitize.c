/*
 * Host-side argument validation and workspace planning of the library, for a
 * build whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer.
 * Every compute call here is rejected by validation before any HIP call (fake,
 * never dereferenced device addresses), so it runs without a GPU; the
 * planners are swept over shapes from the smallest to beyond the limits,
 * where integer overflow would be undefined behaviour.  Test infrastructure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "adamas.h"

#define A ((void *)(uintptr_t)0x10000)   /* aligned fake device address */
#define MIS ((void *)(uintptr_t)0x10001) /* misaligned */

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        printf("FAIL %s: got %d, want %d\n", what, got, want);
        failures++;
    }
}

int main(void)
{
    const int OK = ADAMAS_OK, INV = ADAMAS_ERR_INVALID, UNS = ADAMAS_ERR_UNSUPPORTED,
              WS = ADAMAS_ERR_WORKSPACE;
    expect(adamas_version(), ADAMAS_VERSION, "version");
    for (int s = -3; s < 8; s++)
        if (adamas_status_string(s) == NULL)
            expect(0, 1, "status string");

    /* planners: every op over a grid of shapes (values are not checked here) */
    const int Bs[] = {0, 1, 2, 16, 65535, 65536, 1 << 30};
    const int Hs[][2] = {{1, 1}, {32, 32}, {24, 8}, {8, 1}, {32, 2}, {7, 3}, {65535, 65535},
                         {0, 1}, {1 << 20, 1 << 17}};
    const int64_t ns[] = {-1, 0, 1, 63, 64, 1023, 1024, 1025, 131072, 1 << 20, (int64_t)1 << 31,
                          (int64_t)1 << 40, INT64_MAX};
    const int buds[] = {-1, 0, 1, 64, 256, 1024, 65536, 1 << 20, (1 << 20) + 1, 1 << 30};
    const int dims[] = {0, 63, 64, 96, 128, 256, 512};
    size_t acc = 0;
    long calls = 0;
    for (int op = -1; op < 5; op++)
        for (size_t bi = 0; bi < sizeof Bs / sizeof Bs[0]; bi++)
            for (size_t hi = 0; hi < sizeof Hs / sizeof Hs[0]; hi++)
                for (size_t ni = 0; ni < sizeof ns / sizeof ns[0]; ni++)
                    for (size_t ki = 0; ki < sizeof buds / sizeof buds[0]; ki++)
                        for (size_t di = 0; di < sizeof dims / sizeof dims[0]; di++) {
                            acc += adamas_workspace_bytes(op, Bs[bi], Hs[hi][0], Hs[hi][1],
                                                          ns[ni], buds[ki], dims[di]);
                            if (op == 0)
                                acc += adamas_static_scratch_need(Bs[bi], Hs[hi][0], Hs[hi][1],
                                                                  ns[ni], buds[ki], dims[di]);
                            calls++;
                        }
    for (size_t bytes = 0; bytes < ((size_t)1 << 40); bytes = bytes * 3 + 1)
        acc += adamas_stream_read_blocks(bytes);

    /* encode */
    expect(adamas_encode_keys(A, 0, 1, 1, 4, 96, A, 8, 0, NULL, NULL), UNS, "encode d96");
    expect(adamas_encode_keys(A, 2, 1, 1, 4, 128, A, 8, 0, NULL, NULL), UNS, "encode dtype");
    expect(adamas_encode_keys(A, 1, 1, 1, 4, 128, A, 8, 5, NULL, NULL), INV, "encode pos");
    expect(adamas_encode_keys(A, 1, 1, 1, INT64_MAX, 128, A, 8, 0, NULL, NULL), INV,
           "encode n huge");
    expect(adamas_encode_keys(A, 1, 1, 1, 4, 128, A, INT64_MAX, INT64_MAX, NULL, NULL), INV,
           "encode pos + n overflow");
    expect(adamas_encode_keys(MIS, 1, 1, 1, 4, 128, A, 8, 0, NULL, NULL), INV, "encode align");
    expect(adamas_encode_keys(A, 1, 1, 1, 0, 128, A, 8, 0, NULL, NULL), OK, "encode n=0");

    /* score / select / attend */
    expect(adamas_score(A, A, 1, 8, 3, 128, 1024, 1000, A, NULL), INV, "score Hq%Hkv");
    expect(adamas_score(A, A, 1, 8, 4, 128, 1024, 1025, A, NULL), INV, "score n>cap");
    expect(adamas_score(A, A, 1, 8, 4, 128, INT64_MAX, INT64_MAX, A, NULL), UNS, "score n huge");
    expect(adamas_select_topk(A, 1, 8, 1000, 128, 0, A, A, 1 << 20, NULL), INV, "select b0");
    expect(adamas_select_topk(MIS, 1, 8, 1000, 128, 64, A, A, 1 << 20, NULL), INV,
           "select align");
    expect(adamas_select_topk_keep(A, 1, 8, 1000, 128, 64, -1, 0, A, A, 1 << 20, NULL), INV,
           "select keep sink<0");
    expect(adamas_sparse_attend(A, A, A, 1, A, 1, 8, 4, 128, 1024, 64, NAN, A, A, 1 << 20, NULL),
           INV, "attend nan scale");
    expect(adamas_sparse_attend(A, A, A, 1, A, 1, 8, 4, 128, 1024, 64, 0.0f, A, A, 0, NULL), WS,
           "attend ws");

    /* decode step, its keep and static forms */
    size_t need = adamas_workspace_bytes(ADAMAS_OP_DECODE_STEP, 1, 8, 4, 1000, 64, 128);
    expect(adamas_decode_step(A, A, A, A, 1, 1, 8, 4, 128, 1024, 0, 64, 0.0f, A, NULL, A, need,
                              NULL), INV, "decode n0");
    expect(adamas_decode_step(A, A, A, A, 1, 1, 8, 3, 128, 1024, 1000, 64, 0.0f, A, NULL, A,
                              need, NULL), INV, "decode Hq%Hkv");
    expect(adamas_decode_step(A, A, A, A, 1, 1, 36, 4, 128, 1024, 1000, 64, 0.0f, A, NULL, A,
                              need, NULL), UNS, "decode G9");
    expect(adamas_decode_step(A, A, A, A, 1, 1, 8, 4, 128, 1024, 1000, 64, 0.0f, A, NULL, A,
                              need - 1, NULL), WS, "decode ws");
    expect(adamas_decode_step(A, A, A, MIS, 1, 1, 8, 4, 128, 1024, 1000, 64, 0.0f, A, NULL, A,
                              need, NULL), INV, "decode align");
    expect(adamas_decode_step_keep(A, A, A, A, 1, 1, 8, 4, 128, 1024, 1000, 64, 0, -3, 0.0f, A,
                                   NULL, A, need, NULL), INV, "decode keep recent<0");
    expect(adamas_decode_step_static(A, A, A, A, 1, 1 << 20, 8, 4, 128, 1024, 1000, 64, 0.0f, A,
                                     NULL, NULL), UNS, "static too large");

    /* append and paged steps */
    expect(adamas_decode_append_step(A, A, A, A, A, A, NULL, 1, 2, 8, 4, 128, 1024, 1024, 64, 0, 0,
                                     0.0f, A, NULL, A, 1 << 24, NULL), INV, "append lens null");
    expect(adamas_decode_append_step(A, A, A, A, A, A, A, 1, 2, 8, 4, 128, 1024, 2048, 64, 0, 0,
                                     0.0f, A, NULL, A, 1 << 24, NULL), INV, "append max_len>cap");
    expect(adamas_decode_paged_step(A, A, A, A, A, A, A, A, 1, 2, 8, 4, 128, 1000, 4, 2, 2000, 64,
                                    0, 0, 0.0f, A, NULL, A, 1 << 24, NULL), UNS,
           "paged page size");
    expect(adamas_decode_paged_step(A, A, A, A, A, A, NULL, A, 1, 2, 8, 4, 128, 1024, 4, 2, 2048,
                                    64, 0, 0, 0.0f, A, NULL, A, 1 << 24, NULL), INV,
           "paged table null");

    /* process-wide settings */
    const float good[3] = {0.25f, 0.75f, 0.5f}, bad[2] = {0.5f, -1.0f};
    float back[ADAMAS_MAX_ALPHA_GROUPS];
    expect(adamas_set_bucket_alpha(good, 3), OK, "alpha set");
    expect(adamas_set_bucket_alpha(bad, 2), INV, "alpha negative");
    expect(adamas_set_bucket_alpha(good, ADAMAS_MAX_ALPHA_GROUPS + 1), INV, "alpha n");
    expect(adamas_bucket_alpha(back, 2), 3, "alpha read");
    expect(adamas_set_bucket_alpha(NULL, 0), OK, "alpha reset");
    expect(adamas_set_rotation(3), INV, "rotation 3");
    expect(adamas_set_rotation(1), OK, "rotation 1");
    expect(adamas_set_decode_mode(17), INV, "mode 17");
    expect(adamas_set_wait_polls(0), OK, "polls");
    expect((int)adamas_wait_polls(), 0, "polls read");
    expect(adamas_set_wait_polls(1u << 20), OK, "polls restore");
    expect(adamas_set_phase_buffer(A, 8), adamas_phase_stamps_built() ? INV : UNS,
           "phase buffer");

    printf("host sanitizer run: %ld planner calls (checksum %zu), %d failures\n", calls, acc,
           failures);
    return failures != 0;
}
