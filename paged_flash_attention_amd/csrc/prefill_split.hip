// The KV-split prefill kernel: the prefill of prefill.hip built with 128-row
// workgroups and 32-key tiles (see there).
#define PFA_PREFILL_BN 32
#define PFA_PREFILL_ROWS_WG kPrefillRowsSplit
#define PFA_PREFILL_LAUNCH launch_prefill_split
#include "prefill.hip"
