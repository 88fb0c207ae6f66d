"""CPU oracle for the OTT path: test infrastructure only (see ott_oracle)."""
from .ott_oracle import *  # noqa: F401,F403
from .ott_oracle import (HeadOracle, OTTOracle, Page, pack_page, page_nbytes, run_prefill,
                         softmax, sq_key_norm, step, textbook_attention, min_scale, codes_of,
                         dequant, quantize_members)
