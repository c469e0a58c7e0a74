// Tree-masked attention over a quantised KV cache (gfx950).  Placeholder until the kernel lands.
#include "tv_internal.h"

namespace tv {

size_t attn_workspace_bytes(int, int, int, int, int, int, int) { return 256; }

int launch_attn(const AttnArgs&, hipStream_t) {
    return set_error(TV_EUNSUPPORTED, "attn_tree_verify: kernel not built yet");
}

}  // namespace tv
