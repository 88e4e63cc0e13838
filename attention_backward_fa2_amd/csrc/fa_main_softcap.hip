// fa_main_softcap.hip -- the soft-capped instantiations (scores c * tanh(x /
// c), mha_bwd's softcap on the backward call-trace page) of the key-tile
// kernel of fa_main.hip, in a translation unit of their own so that they
// compile in parallel with the rest.
#define FA_TU_SOFTCAP 1
#include "fa_main.hip"
