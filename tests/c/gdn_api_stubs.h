/* gdn_api_stubs.h - what the host-only launcher stubs (gdn_api_stubs.cpp)
 * record of each launch the C-ABI layer makes, for the sanitizer check of
 * that layer (gdn_api_check.c).  Test infrastructure only. */
#ifndef GDN_API_STUBS_H
#define GDN_API_STUBS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STUB_MAX_LAUNCHES 16

/* One recorded launch.  kind: "step", "seq", "seq_exact", "pair",
 * "tail_fused", "tail_pair", "prestate", "gated_norm" or "gate".
 * p[], i[], l[] and f hold the launcher's arguments in the order the stubs
 * list them. */
typedef struct {
    char kind[16];
    const void *p[16];
    int32_t i[8];
    int64_t l[2];
    float f;
    const void *stream;
} stub_launch;

void stub_reset(void);
/* The index-th launch from now (0: the next) reports hipErrorLaunchFailure. */
void stub_fail_launch(int index);
int stub_n_launches(void);
const stub_launch *stub_launch_at(int i);
int stub_scratch_lookups(void);
const void *stub_scratch(void);
size_t stub_scratch_bytes(void);
int stub_tail_fused_supported(int32_t Hv, int32_t Hk, int32_t K, int32_t group);

#ifdef __cplusplus
}
#endif

#endif
