/*
 * Calls every entry point of include/rsu.h with arguments that fail validation (a NULL
 * dims or array, dims other than 128 x 128, a misaligned array, an out-of-range window,
 * log length or sub-step count) or with an empty batch, for a build of the library with
 * the host address and undefined-behaviour sanitizers: the validation and error-reporting
 * paths run without touching a GPU (no call passes validation with a non-empty batch).
 * Exits 0 when every call returns the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rsu.h"

#define G ((void *)0x1000) /* aligned, never dereferenced */
#define O ((void *)0x1004) /* misaligned */

static int fails = 0;
static void expect(const char *what, int got, int want, const char *msg_part) {
    const char *msg = rsu_last_error();
    if (got != want || (msg_part && !strstr(msg, msg_part))) {
        fprintf(stderr, "%s: got %d (\"%s\"), want %d%s%s\n", what, got, msg, want, msg_part ? " with " : "",
                msg_part ? msg_part : "");
        fails++;
    }
}

int main(void) {
    rsu_dims d = {2, 3, 128, 128, RSU_BF16}, bad = {2, 3, 128, 64, RSU_BF16}, e = {0, 3, 128, 128, RSU_BF16};
    rsu_dims dt = {2, 3, 128, 128, 7}, neg = {-1, 3, 128, 128, RSU_F32};
    float *f = (float *)G, *fo = (float *)O;
    int8_t *z = (int8_t *)G;

    expect("version", rsu_abi_version(), 1, NULL);
    expect("dense null dims", gdn_decode_step(NULL, f, G, G, G, f, f, f, NULL), RSU_E_NULL, "dims is NULL");
    expect("dense dims", gdn_decode_step(&bad, f, G, G, G, f, f, f, NULL), RSU_E_DIMS, "dv=64");
    expect("dense dtype", kda_decode_step(&dt, f, G, G, G, f, f, f, NULL), RSU_E_DTYPE, "qkv_dtype=7");
    expect("dense negative", kda_decode_step(&neg, f, G, G, G, f, f, f, NULL), RSU_E_DIMS, NULL);
    expect("dense null S", gdn_decode_step(&d, NULL, G, G, G, f, f, f, NULL), RSU_E_NULL, "S is NULL");
    expect("dense align", kda_decode_step(&d, f, G, O, G, f, f, f, NULL), RSU_E_ALIGN, "k is not 16-byte");
    expect("dense empty", gdn_decode_step(&e, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), RSU_OK, NULL);
    expect("rwkv6 null w", rwkv6_decode_step(&d, f, G, G, G, NULL, f, NULL), RSU_E_NULL, "w is NULL");
    expect("rwkv7 null a", rwkv7_decode_step(&d, f, G, G, G, G, f, NULL, f, NULL), RSU_E_NULL, "a is NULL");
    expect("dp n", deltaproduct_decode_step(&d, 5, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, "n=5");
    expect("dp align", deltaproduct_decode_step(&d, 2, f, G, G, G, fo, f, f, NULL), RSU_E_ALIGN, "alpha");

    expect("quantize null", q8_quantize(&d, f, NULL, f, NULL), RSU_E_NULL, "Z is NULL");
    expect("window W", gdn_q8_window(&d, 33, 0, z, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, "W=33");
    expect("window pos", kda_q8_window(&d, 16, 16, z, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, "pos=16");
    expect("window null", gdn_q8_window(&d, 16, 3, z, f, G, NULL, f, G, G, G, f, f, f, NULL), RSU_E_NULL, "Ubuf");
    expect("rwkv7 window W", rwkv7_q8_window(&d, 17, 0, z, f, G, f, f, G, G, G, G, f, f, f, NULL), RSU_E_RANGE, NULL);
    expect("dp window nW", deltaproduct_q8_window(&d, 2, 17, 0, z, f, G, f, f, G, G, G, f, f, f, NULL),
           RSU_E_RANGE, "n W");
    expect("dp window empty", deltaproduct_q8_window(&e, 2, 16, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                                     NULL, NULL, NULL, NULL), RSU_OK, NULL);

    expect("log append L", gdn_log_append(&d, 7, 7, f, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, "L=7");
    expect("log merge L", kda_log_merge(&d, 7, 6, f, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, NULL);
    expect("log C", gdn_log_merge(&d, 64, 64, f, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, "C=64");
    expect("log null log", gdn_log_append(&d, 7, 0, f, f, NULL, f, f, G, G, G, f, f, f, NULL), RSU_E_NULL, "Klog");
    expect("log C=0", gdn_log_merge(&d, 0, 0, f, f, NULL, NULL, NULL, G, G, G, f, f, NULL, NULL), RSU_E_NULL, "y");
    expect("kda append", kda_log_append(&d, 7, 7, f, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, "L=7");
    expect("gdn slots", gdn_log_step_slots(&d, 7, NULL, f, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_NULL, NULL);
    expect("slots null L", kda_log_step_slots(&d, 7, NULL, f, f, G, f, f, G, G, G, f, f, f, NULL), RSU_E_NULL, "L is");
    expect("rwkv6 log", rwkv6_log_append(&d, 3, 3, f, f, G, G, f, G, G, G, f, f, NULL), RSU_E_RANGE, NULL);
    expect("rwkv6 merge", rwkv6_log_merge(&d, 3, 2, f, f, G, G, f, G, G, G, f, f, NULL), RSU_E_RANGE, NULL);
    expect("rwkv6 slots", rwkv6_log_step_slots(&d, 3, NULL, f, f, G, G, f, G, G, G, f, f, NULL), RSU_E_NULL, NULL);

    rsu_dims df = {2, 3, 128, 128, RSU_F32};
    expect("lq dtype", gdn_lq_window(&df, 16, 0, 1, z, f, f, G, G, G, f, f, G, G, G, f, f, f, NULL), RSU_E_DTYPE,
           "bf16");
    expect("lq W", kda_lq_window(&d, 17, 0, 1, z, f, f, G, G, G, f, f, G, G, G, f, f, f, NULL), RSU_E_RANGE, NULL);
    expect("lq n_iter", gdn_lq_quantize(&d, f, 65, z, f, f, G, G, NULL), RSU_E_RANGE, "n_iter=65");
    expect("lq4 null", gdn_lq4_window(&d, 16, 0, 1, G, f, f, NULL, G, G, f, f, G, G, G, f, f, f, NULL), RSU_E_NULL,
           "Kc");
    expect("lq4 quantize", gdn_lq4_quantize(&d, NULL, 1, G, f, f, G, G, NULL), RSU_E_NULL, "S is NULL");
    expect("kda lq quantize", kda_lq_quantize(&bad, f, 1, z, f, f, G, G, NULL), RSU_E_DIMS, NULL);

    expect("stepq pack", stepq_pack(&d, f, NULL, G, G, G, NULL), RSU_E_NULL, "omega");
    expect("stepq step", gdn_stepq_step(&d, G, G, G, f, G, G, G, f, f, NULL, NULL), RSU_E_NULL, "y is NULL");
    expect("stepq kda", kda_stepq_step(&d, O, G, G, f, G, G, G, f, f, f, NULL), RSU_E_ALIGN, "Z is not");
    expect("stepq readout", gdn_stepq_readout(&d, G, G, G, G, G, G, f, f, NULL, f, NULL), RSU_E_NULL, "u is NULL");
    expect("stepq kda readout", kda_stepq_readout(&bad, G, G, G, G, G, G, f, f, f, f, NULL), RSU_E_DIMS, NULL);
    expect("stepq repack", gdn_stepq_repack(&d, G, G, G, f, G, f, NULL, NULL), RSU_E_NULL, "u is NULL");
    expect("stepq kda repack", kda_stepq_repack(&e, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), RSU_OK, NULL);

    uint32_t counts[8 * 4];
    expect("counts null", rsu_debug_metadata_counts(NULL, 4, NULL), RSU_E_NULL, "counts");
    expect("counts heads", rsu_debug_metadata_counts(counts, 65537, NULL), RSU_E_RANGE, "heads=65537");
    expect("counts build", rsu_debug_metadata_counts(counts, 4, NULL), RSU_E_UNSUPPORTED, "RSU_CHECK_METADATA");

    expect("copy n", rsu_copy_f32(f, f, 6, NULL), RSU_E_DIMS, "multiple of 4");
    expect("read tiles", rsu_read_f32(f, f, -1, NULL), RSU_E_DIMS, NULL);
    expect("fill align", rsu_fill_f32(fo, 1.f, 2, NULL), RSU_E_ALIGN, NULL);
    expect("copy empty", rsu_copy_f32(NULL, NULL, 0, NULL), RSU_OK, NULL);

    if (fails == 0) printf("abi driver ok\n");
    return fails != 0;
}
